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
//   uses DPP row_shr 1/2/4/8 inside 16-lane rows and row_bcast 15/31 across rows.  DPP has
//   no broadcast towards lower lanes, so a suffix scan over the wave runs as a forward scan in
//   reversed lane order (ds_bpermute reverses the wave), or, in the complex kernels, as row_shl
//   levels inside rows and readlane across rows.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "msel_kernels.hpp"

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

// ---------------------------------------------------------------------------------------
// Bounds checks of the checked build.  Built with -DMSEL_CHECKED (libmsel_checked.so), every
// index that a kernel forms into a global buffer or an LDS array goes through MSEL_IDX(i, n),
// n being the extent of what it indexes (for a row, the number of rows).  An index outside
// [0, n) is counted in its source file's device record (with the source line of the first one),
// which the host reads and clears, and is replaced by 0: the access then stays inside the
// buffer and the kernel ends normally, so a failed check never traps, faults or hangs.
// Without MSEL_CHECKED, MSEL_IDX(i, n) is i, and MSEL_BOUNDS_TAKER defines a reader of an
// empty record.  Row accesses through buffer resources are range-checked by the hardware
// within the row; their row index is what MSEL_IDX checks.
#ifdef MSEL_CHECKED
static __device__ BoundsRecord g_bounds;  // one per source file

template <typename I>
__device__ __forceinline__ I checked_index(I i, unsigned long long n, unsigned int line) {
    if (static_cast<long long>(i) >= 0 && static_cast<unsigned long long>(i) < n) return i;
    if (__hip_atomic_fetch_add(&g_bounds.count, 1ull, __ATOMIC_RELAXED,
                               __HIP_MEMORY_SCOPE_AGENT) == 0)
        __hip_atomic_store(&g_bounds.line, line, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    return I(0);
}
#define MSEL_IDX(i, n) ::msel::checked_index((i), static_cast<unsigned long long>(n), __LINE__)
#define MSEL_BOUNDS_TAKER(fn)                                                                  \
    hipError_t fn(::msel::BoundsRecord* out) {                                                 \
        const ::msel::BoundsRecord zero{};                                                     \
        hipError_t e = hipMemcpyFromSymbol(out, HIP_SYMBOL(::msel::g_bounds), sizeof(*out), 0, \
                                           hipMemcpyDeviceToHost);                             \
        if (e == hipSuccess)                                                                   \
            e = hipMemcpyToSymbol(HIP_SYMBOL(::msel::g_bounds), &zero, sizeof(zero), 0,        \
                                  hipMemcpyHostToDevice);                                      \
        return e;                                                                              \
    }
#else
#define MSEL_IDX(i, n) (i)
#define MSEL_BOUNDS_TAKER(fn)                      \
    hipError_t fn(::msel::BoundsRecord* out) {     \
        *out = ::msel::BoundsRecord{};             \
        return hipSuccess;                         \
    }
#endif

__device__ __forceinline__ float sigmoid_f(float x) { return rcp_hw(1.0f + exp2_hw(-x * kLog2e)); }

// The softplus's derivative sigmoid(x), given x and its softplus sp = log(1 + e^x):
// sigmoid(x) = e^x / (1 + e^x) = exp(x - sp), one exp.  (The other one-exp form, 1 - exp(-sp),
// cancels for small sp: at sp = 1e-4 it keeps only ~4 significant digits.)  x - sp = -log(1 +
// e^-x) is exact where it is large, and where it is tiny (x large) the sigmoid is ~1 anyway.
__device__ __forceinline__ float softplus_grad_f(float x, float sp) {
    return exp2_hw((x - sp) * kLog2e);
}

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

// Lane l's element of a wave-uniform row of n floats, through the row's buffer resource: lanes
// at or past n read 0 and store nothing.  The address stays the row's scalar base plus the
// lane's byte offset, so no 64-bit address per lane is kept in registers.
__device__ __forceinline__ float load_lane(const float* row, int n, int lane) {
    return __uint_as_float(__builtin_amdgcn_raw_buffer_load_b32(row_rsrc(row, n), lane * 4, 0, 0));
}
__device__ __forceinline__ void store_lane(float* row, int n, int lane, float v) {
    __builtin_amdgcn_raw_buffer_store_b32(__float_as_uint(v), row_rsrc(row, n), lane * 4, 0, 0);
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

// Rows of one tile (64*K steps) staged in LDS as fp32 by a whole workgroup of NTH threads and
// read by each of its wavefronts: for rows shared by the workgroup's channels (B and C of one
// batch row), which are then loaded and converted once per workgroup instead of once per
// wavefront.  A buffer is [ROWS rows][K/4 words][64 lanes (+2 padding)] of 16-byte words, so
// that lane l reads its K steps of a row as K/4 words of its own column, the 64 lanes
// consecutive words.
// load() issues the global loads of one set of rows into registers (thread tid moves vectors
// tid, tid + NTH, ...; a row is a whole number of wavefronts' vectors, so which row a vector
// belongs to is wave-uniform); store() converts them into a buffer; read() gives a lane its K
// values of one row.  The caller separates a store and the reads of the same buffer by a
// workgroup barrier.
template <typename T, int K, int ROWS, int NTH, bool VEC>
struct TileStage {
    static constexpr int QW = K / 4;                 // 16-byte words per lane and row
    static constexpr int VW = Elem<T>::kPerVec;      // elements per 16-byte vector
    static constexpr int RV = 64 * K / VW;           // vectors per row
    static constexpr int NVEC = ROWS * RV;
    static constexpr int G = (NVEC + NTH - 1) / NTH; // vectors per thread (the last partial)
    // 16-byte words from one (row, word) line of 64 lanes to the next: 66, not 64.  A store
    // pass (8 lanes, 128 bytes) puts neighbouring threads' vectors in different lines of the
    // same lane (fp32: 4 lines of one lane; bf16: 2 lines of each of 4 lanes); with lines
    // 2 words (32 bytes) apart modulo 128 bytes, those 8 vectors fill 8 different bank groups.
    // Reads stay 64 consecutive words of one line.
    static constexpr int kLine = 64 + 2;
    static constexpr int kWords = ROWS * QW * kLine; // 16-byte words per buffer
    static_assert(K % VW == 0 && K % 4 == 0 && RV % 64 == 0 && NTH % 64 == 0,
                  "a row must split over whole wavefronts");
    Raw<T, VW> nxt[G];
    int xr[G];    // staged row of this thread's i-th vector (wave-uniform)
    int toff[G];  // its first step within the tile

    __device__ __forceinline__ explicit TileStage(int tid) {
#pragma unroll
        for (int i = 0; i < G; ++i) {
            const int v = tid + i * NTH;
            xr[i] = __builtin_amdgcn_readfirstlane(v / RV);
            toff[i] = (v - xr[i] * RV) * VW;
        }
    }

    // row(x): the global row that staged row x comes from; t_tile: the tile's first step
    template <typename RowFn>
    __device__ __forceinline__ void load(int tid, RowFn row, int t_tile, int L) {
#pragma unroll
        for (int i = 0; i < G; ++i) {
            if (NVEC % NTH != 0 && tid + i * NTH >= NVEC) break;  // wave-uniform
            load_raw<T, VW, VEC>(row(xr[i]), t_tile + toff[i], L, nxt[i]);
        }
    }
    __device__ __forceinline__ void store(int tid, f32x4* __restrict__ buf) const {
#pragma unroll
        for (int i = 0; i < G; ++i) {
            const int v = tid + i * NTH;
            if (NVEC % NTH != 0 && v >= NVEC) break;
            const int x = v / RV;
            const int tl = (v - x * RV) * VW;
            float f[VW];
            unpack<T, VW>(nxt[i], f);
            const int l = tl / K, q0 = (tl - l * K) / 4;
#pragma unroll
            for (int j = 0; j < VW / 4; ++j)
                buf[MSEL_IDX((x * QW + q0 + j) * kLine + l, kWords)] =
                    f32x4{f[4 * j], f[4 * j + 1], f[4 * j + 2], f[4 * j + 3]};
        }
    }
    __device__ __forceinline__ static void read(const f32x4* __restrict__ buf, int x, int lane,
                                                float (&r)[K]) {
#pragma unroll
        for (int q = 0; q < QW; ++q) {
            const f32x4 w4 = buf[MSEL_IDX((x * QW + q) * kLine + lane, kWords)];
            r[4 * q] = w4[0];
            r[4 * q + 1] = w4[1];
            r[4 * q + 2] = w4[2];
            r[4 * q + 3] = w4[3];
        }
    }
};

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
// Lane `lane` of the result is v, the other lanes keep old: one v_writelane_b32.  v and lane
// must be wave-uniform (every caller passes a readlane result or a wave-wide sum).  gfx9
// reads at most one SGPR per VALU instruction through the constant bus, so the lane select
// goes in M0.
__device__ __forceinline__ float writelane(float v, int lane, float old) {
    asm("v_writelane_b32 %0, %1, m0" : "+v"(old) : "s"(v), "{m0}"(lane));
    return old;
}

__device__ __forceinline__ int lane_id() { return __lane_id(); }


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

// Two independent inclusive forward scans over the 64 lanes in one instruction stream.  Each
// DPP read comes at least three instructions after the write of its source, so the levels need
// no wait states (only the first, after the inputs were written).
__device__ __forceinline__ void scan_fwd2_fused(float& P, float& S, float& P2, float& S2) {
#define MSEL_FWD2_LEVEL(CTRL, RMASK)                                                 \
    "v_fmac_f32_dpp %[S], %[S], %[P] " CTRL " row_mask:" RMASK " bank_mask:0xf\n"      \
    "v_mul_f32_dpp %[P], %[P], %[P] " CTRL " row_mask:" RMASK " bank_mask:0xf\n"       \
    "v_fmac_f32_dpp %[S2], %[S2], %[P2] " CTRL " row_mask:" RMASK " bank_mask:0xf\n"   \
    "v_mul_f32_dpp %[P2], %[P2], %[P2] " CTRL " row_mask:" RMASK " bank_mask:0xf\n"
    asm volatile("s_nop 1\n"
                 MSEL_FWD2_LEVEL("row_shr:1", "0xf")
                 MSEL_FWD2_LEVEL("row_shr:2", "0xf")
                 MSEL_FWD2_LEVEL("row_shr:4", "0xf")
                 MSEL_FWD2_LEVEL("row_shr:8", "0xf")
                 MSEL_FWD2_LEVEL("row_bcast:15", "0xa")
                 MSEL_FWD2_LEVEL("row_bcast:31", "0xc")
                 : [P] "+v"(P), [S] "+v"(S), [P2] "+v"(P2), [S2] "+v"(S2));
#undef MSEL_FWD2_LEVEL
}

// The value of lane 63 - l in lane l (a whole-wave reversal through the LDS crossbar, no LDS
// memory); rev_addr is (63 - lane) * 4.
__device__ __forceinline__ float rev_lanes(float v, int rev_addr) {
    return __builtin_bit_cast(float, __builtin_amdgcn_ds_bpermute(rev_addr, __builtin_bit_cast(int, v)));
}

// Sum over each group of four consecutive lanes (every lane of the group gets it): two DPP
// adds (the wait states before each DPP read of a VGPR written just before are the s_nops).
__device__ __forceinline__ float quad_sum(float v) {
    asm("s_nop 1\n"
        "v_add_f32_dpp %0, %0, %0 quad_perm:[1,0,3,2] row_mask:0xf bank_mask:0xf\n"
        "s_nop 1\n"
        "v_add_f32_dpp %0, %0, %0 quad_perm:[2,3,0,1] row_mask:0xf bank_mask:0xf\n"
        : "+v"(v));
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

// Sum of v over the lanes before this one (lane 0 gets 0).
__device__ __forceinline__ float wave_excl_sum(float v) { return shift_up(wave_incl_sum(v), 0.0f); }

// Sum of v over the lanes after this one (lane 63 gets 0): the exclusive prefix sum in
// reversed lane order (rev_addr = (63 - lane) * 4).  Partial sums of step sizes are always
// formed this way, as sums of the terms they cover: a difference of two totals, such as
// total - prefix, loses the small remainder next to one huge step (a state reset, whose
// Delta * A is hundreds), and exp(A * remainder) then carries that error.
__device__ __forceinline__ float wave_excl_suffix_sum(float v, int rev_addr) {
    return rev_lanes(wave_excl_sum(rev_lanes(v, rev_addr)), rev_addr);
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

// ---------------------------------------------------------------------------------------
// Complex states as (Re, Im) pairs of fp32 (the rotational variant).

constexpr float kInv2Pi = 0.15915494309189535f;

// sin and cos of an angle given in revolutions: v_sin_f32 / v_cos_f32 take revolutions, and
// reducing to [0, 1) first keeps any step size inside their input range.
__device__ __forceinline__ float sin_rev(float r) {
    return __builtin_amdgcn_sinf(__builtin_amdgcn_fractf(r));
}
__device__ __forceinline__ float cos_rev(float r) {
    return __builtin_amdgcn_cosf(__builtin_amdgcn_fractf(r));
}

// r + i i = (ar + i ai)(br + i bi)
__device__ __forceinline__ void cmul(float ar, float ai, float br, float bi, float& r, float& i) {
    r = fmaf(ar, br, -ai * bi);
    i = fmaf(ar, bi, ai * br);
}

// Scans of complex affine pairs over the lanes: (P, S) <- (P Q, P T + S), (Q, T) the pair of
// the DPP source lane, with the DPP moves fused into the arithmetic as in the real scans above
// (a lane without a source is not written: the identity).  A level reads the source's Q and
// T while this lane's P and S are being replaced, so it first copies S_im, P_re and P_im
// (cs, cr, ci), then, with src0 the source lane's value:
//   S_im += T_re P_im   S_re += T_re P_re   P_re = Q_re P_re   P_im = Q_re P_im
//   S_im += T_im P_re   S_re -= T_im P_im   P_re -= Q_im P_im  P_im += Q_im P_re
// S_re is read through DPP before it is written; every DPP read of a register comes at least
// two instructions after its write (the copies lead, and the next level's DPP read of S_re
// follows five instructions after this level's write), so no s_nop is needed.
#define MSEL_CPLX_LEVEL(CTRL, RMASK, PR, PI, SR, SI)                                        \
    "v_mov_b32 %[cs], %[" SI "]\n"                                                          \
    "v_mov_b32 %[cr], %[" PR "]\n"                                                          \
    "v_mov_b32 %[ci], %[" PI "]\n"                                                          \
    "v_fmac_f32_dpp %[" SI "], %[" SR "], %[ci] " CTRL " row_mask:" RMASK " bank_mask:0xf\n" \
    "v_fmac_f32_dpp %[" SR "], %[" SR "], %[cr] " CTRL " row_mask:" RMASK " bank_mask:0xf\n" \
    "v_mul_f32_dpp %[" PR "], %[cr], %[cr] " CTRL " row_mask:" RMASK " bank_mask:0xf\n"      \
    "v_mul_f32_dpp %[" PI "], %[cr], %[ci] " CTRL " row_mask:" RMASK " bank_mask:0xf\n"      \
    "v_fmac_f32_dpp %[" SI "], %[cs], %[cr] " CTRL " row_mask:" RMASK " bank_mask:0xf\n"     \
    "v_fmac_f32_dpp %[" SR "], %[cs], -%[ci] " CTRL " row_mask:" RMASK " bank_mask:0xf\n"    \
    "v_fmac_f32_dpp %[" PR "], %[ci], -%[ci] " CTRL " row_mask:" RMASK " bank_mask:0xf\n"    \
    "v_fmac_f32_dpp %[" PI "], %[ci], %[cr] " CTRL " row_mask:" RMASK " bank_mask:0xf\n"

// Inclusive scan over the 64 lanes, lane 0 first.
__device__ __forceinline__ void cscan_fused(float& Pr, float& Pi, float& Sr, float& Si) {
    float cs, cr, ci;
    asm volatile(MSEL_CPLX_LEVEL("row_shr:1", "0xf", "Pr", "Pi", "Sr", "Si")
                 MSEL_CPLX_LEVEL("row_shr:2", "0xf", "Pr", "Pi", "Sr", "Si")
                 MSEL_CPLX_LEVEL("row_shr:4", "0xf", "Pr", "Pi", "Sr", "Si")
                 MSEL_CPLX_LEVEL("row_shr:8", "0xf", "Pr", "Pi", "Sr", "Si")
                 MSEL_CPLX_LEVEL("row_bcast:15", "0xa", "Pr", "Pi", "Sr", "Si")
                 MSEL_CPLX_LEVEL("row_bcast:31", "0xc", "Pr", "Pi", "Sr", "Si")
                 : [Pr] "+v"(Pr), [Pi] "+v"(Pi), [Sr] "+v"(Sr), [Si] "+v"(Si), [cs] "=&v"(cs),
                   [cr] "=&v"(cr), [ci] "=&v"(ci));
}

// The same forward scan of (P, S) and, in one instruction stream, the suffix composition of
// (R, T) within each 16-lane row (row_shl: each lane composes the lanes after it in its row).
__device__ __forceinline__ void cscan2_fused(float& Pr, float& Pi, float& Sr, float& Si,
                                             float& Rr, float& Ri, float& Tr, float& Ti) {
    float cs, cr, ci;
    asm volatile(MSEL_CPLX_LEVEL("row_shr:1", "0xf", "Pr", "Pi", "Sr", "Si")
                 MSEL_CPLX_LEVEL("row_shl:1", "0xf", "Rr", "Ri", "Tr", "Ti")
                 MSEL_CPLX_LEVEL("row_shr:2", "0xf", "Pr", "Pi", "Sr", "Si")
                 MSEL_CPLX_LEVEL("row_shl:2", "0xf", "Rr", "Ri", "Tr", "Ti")
                 MSEL_CPLX_LEVEL("row_shr:4", "0xf", "Pr", "Pi", "Sr", "Si")
                 MSEL_CPLX_LEVEL("row_shl:4", "0xf", "Rr", "Ri", "Tr", "Ti")
                 MSEL_CPLX_LEVEL("row_shr:8", "0xf", "Pr", "Pi", "Sr", "Si")
                 MSEL_CPLX_LEVEL("row_shl:8", "0xf", "Rr", "Ri", "Tr", "Ti")
                 MSEL_CPLX_LEVEL("row_bcast:15", "0xa", "Pr", "Pi", "Sr", "Si")
                 MSEL_CPLX_LEVEL("row_bcast:31", "0xc", "Pr", "Pi", "Sr", "Si")
                 : [Pr] "+v"(Pr), [Pi] "+v"(Pi), [Sr] "+v"(Sr), [Si] "+v"(Si), [Rr] "+v"(Rr),
                   [Ri] "+v"(Ri), [Tr] "+v"(Tr), [Ti] "+v"(Ti), [cs] "=&v"(cs), [cr] "=&v"(cr),
                   [ci] "=&v"(ci));
}
#undef MSEL_CPLX_LEVEL

}  // namespace msel
