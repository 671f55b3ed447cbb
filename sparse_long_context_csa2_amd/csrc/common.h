// Internal definitions shared by the CSA2 HIP kernels and the C-ABI host code.
// Target: gfx950 (CDNA4), wave64.
#pragma once

#include <hip/hip_runtime.h>

#include <cstddef>
#include <cstdint>
#include <stdexcept>
#include <string>

#include "../../include/csa2.h"

namespace csa2 {

// ------------------------------------------------------------------ vectors
typedef __bf16 bf16;
typedef __attribute__((__vector_size__(8 * sizeof(__bf16)))) __bf16 bf16x8;
typedef __attribute__((__vector_size__(8 * sizeof(_Float16)))) _Float16 f16x8;
typedef __attribute__((__vector_size__(4 * sizeof(float)))) float f32x4;
typedef __attribute__((__vector_size__(4 * sizeof(uint32_t)))) uint32_t u32x4;
typedef __attribute__((__vector_size__(2 * sizeof(__bf16)))) __bf16 bf16x2;
typedef short __attribute__((ext_vector_type(2))) s16x2;

constexpr int WAVE = 64;

// ------------------------------------------------------------ host errors
struct Error : std::runtime_error {
    int code;
    Error(int c, const std::string &m) : std::runtime_error(m), code(c) {}
};

#define CSA2_REQUIRE(cond, code, msg)                                      \
    do {                                                                   \
        if (!(cond)) throw ::csa2::Error((code), std::string(msg));       \
    } while (0)

#define CSA2_HIP(call)                                                                 \
    do {                                                                               \
        hipError_t e_ = (call);                                                        \
        if (e_ != hipSuccess)                                                          \
            throw ::csa2::Error(CSA2_EHIP, std::string(#call ": ") + hipGetErrorString(e_)); \
    } while (0)

inline void check_launch(const char *what) {
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) throw Error(CSA2_EHIP, std::string(what) + ": " + hipGetErrorString(e));
}

// ------------------------------------------------------------- workspace
// Bump allocator over the caller's workspace; every block is 256-byte aligned.
struct Carve {
    char *base;
    size_t cap, used = 0;
    explicit Carve(void *b, size_t c) : base(static_cast<char *>(b)), cap(c) {}
    template <class T>
    T *take(size_t count) {
        size_t bytes = (count * sizeof(T) + 255) & ~size_t(255);
        T *p = base ? reinterpret_cast<T *>(base + used) : nullptr;
        used += bytes;
        return p;
    }
};

// ------------------------------------------------------------ device bits
// FP4 row scale byte (E4M3FN: bias 7, exponent field 0 = m 2^-9) -> its
// magnitude as binary32 bits, the NaN code S.1111.111 taken as 448 = 2^8 x 1.75
// (one corrupt byte must not turn a row into NaNs).  Both encodings are formed
// and one is selected, so the decode has no branch: written as a conditional
// value it compiled to a divergent branch per scale byte.
__device__ __forceinline__ uint32_t e4m3_mag_bits(uint32_t sbyte) {
    const uint32_t e = (sbyte >> 3) & 15u;
    const uint32_t m = (sbyte & 0x7fu) == 0x7fu ? 6u : (sbyte & 7u);
    const uint32_t nbits = ((e + 120u) << 23) | (m << 20);           // exponent field >= 1
    const uint32_t sbits = __float_as_uint((float)m * 0.001953125f);  // exponent field 0
    return e ? nbits : sbits;
}

__device__ __forceinline__ float bf16_to_f32(uint16_t h) { return __uint_as_float(uint32_t(h) << 16); }

// Round-to-nearest-even fp32 -> bf16 bits (inputs are finite).
__device__ __forceinline__ uint16_t f32_to_bf16_rne(float f) {
    uint32_t u = __float_as_uint(f);
    u += 0x7fffu + ((u >> 16) & 1u);
    return uint16_t(u >> 16);
}

// ------------------------------------------------------- cross-lane steps
// Butterfly steps on 32-bit lanes without the LDS crossbar: DPP for partners
// inside a 16-lane row, the gfx950 permlane swaps across rows.  bfly_k(v, op)
// returns op(v, v of lane l ^ k) in every lane (op commutative), except that
// bfly4 / bfly8 pair lane l with l ^ 7 / l ^ 15 (row half-mirror / mirror):
// the same as l ^ 4 / l ^ 8 once the smaller steps have made groups of 4 / 8
// lanes equal, which is how the reductions below use them.
template <int CTRL>
__device__ __forceinline__ uint32_t dpp(uint32_t v) {
    return (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, CTRL, 0xF, 0xF, false);
}
template <class T>
__device__ __forceinline__ uint32_t as_u32(T v) { return __builtin_bit_cast(uint32_t, v); }
template <class T>
__device__ __forceinline__ T from_u32(uint32_t v) { return __builtin_bit_cast(T, v); }

template <class T, class Op>
__device__ __forceinline__ T bfly1(T v, Op op) { return op(v, from_u32<T>(dpp<0xB1>(as_u32(v)))); }
template <class T, class Op>
__device__ __forceinline__ T bfly2(T v, Op op) { return op(v, from_u32<T>(dpp<0x4E>(as_u32(v)))); }
template <class T, class Op>
__device__ __forceinline__ T bfly4(T v, Op op) { return op(v, from_u32<T>(dpp<0x141>(as_u32(v)))); }
template <class T, class Op>
__device__ __forceinline__ T bfly8(T v, Op op) { return op(v, from_u32<T>(dpp<0x140>(as_u32(v)))); }
template <class T, class Op>
__device__ __forceinline__ T bfly16(T v, Op op) {
    const auto r = __builtin_amdgcn_permlane16_swap(as_u32(v), as_u32(v), false, false);
    return op(from_u32<T>(r[0]), from_u32<T>(r[1]));
}
template <class T, class Op>
__device__ __forceinline__ T bfly32(T v, Op op) {
    const auto r = __builtin_amdgcn_permlane32_swap(as_u32(v), as_u32(v), false, false);
    return op(from_u32<T>(r[0]), from_u32<T>(r[1]));
}
template <class T, class Op>
__device__ __forceinline__ T wave_reduce(T v, Op op) {
    v = bfly1(v, op);
    v = bfly2(v, op);
    v = bfly4(v, op);
    v = bfly8(v, op);
    v = bfly16(v, op);
    return bfly32(v, op);
}
struct OpAdd {
    template <class T>
    __device__ T operator()(T a, T b) const { return a + b; }
};
struct OpMax {
    __device__ float operator()(float a, float b) const { return fmaxf(a, b); }
};
struct OpMin {
    __device__ float operator()(float a, float b) const { return fminf(a, b); }
};
struct OpMaxU {
    __device__ uint32_t operator()(uint32_t a, uint32_t b) const { return a > b ? a : b; }
};

// Inclusive prefix sum over the 64 lanes: shifts by 1, 2, 4, 8 inside each
// 16-lane row, then the row totals are carried forward with the row
// broadcasts of lane 15 (into rows 1 and 3) and lane 31 (into rows 2 and 3).
// Lanes that a shift or broadcast does not reach add 0.
__device__ __forceinline__ uint32_t wave_incl_scan_u32(uint32_t v) {
    v += (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0x111, 0xF, 0xF, false);  // row_shr:1
    v += (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0x112, 0xF, 0xF, false);  // row_shr:2
    v += (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0x114, 0xF, 0xF, false);  // row_shr:4
    v += (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0x118, 0xF, 0xF, false);  // row_shr:8
    v += (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0x142, 0xA, 0xF, false);  // row_bcast:15
    v += (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0x143, 0xC, 0xF, false);  // row_bcast:31
    return v;
}

__device__ __forceinline__ float wave_sum(float v) { return wave_reduce(v, OpAdd{}); }
__device__ __forceinline__ float wave_max(float v) { return wave_reduce(v, OpMax{}); }
__device__ __forceinline__ float wave_min(float v) { return wave_reduce(v, OpMin{}); }
__device__ __forceinline__ uint32_t wave_sum_u32(uint32_t v) { return wave_reduce(v, OpAdd{}); }
__device__ __forceinline__ uint32_t wave_max_u32(uint32_t v) { return wave_reduce(v, OpMaxU{}); }

// Order-preserving key of a binary64 value (-0 is folded onto +0 so that it
// ties with +0, as numeric comparison does).
__device__ __forceinline__ uint64_t dkey(double d) {
    if (d == 0.0) d = 0.0;
    uint64_t u = __double_as_longlong(d);
    return (u >> 63) ? ~u : (u | 0x8000000000000000ull);
}
__device__ __forceinline__ double dkey_inv(uint64_t k) {
    uint64_t u = (k >> 63) ? (k & 0x7fffffffffffffffull) : ~k;
    return __longlong_as_double(u);
}
// Order-preserving key of a binary32 value over the finite range.
__device__ __forceinline__ uint32_t fkey(float f) {
    if (f == 0.0f) f = 0.0f;
    uint32_t u = __float_as_uint(f);
    return (u >> 31) ? ~u : (u | 0x80000000u);
}
__device__ __forceinline__ float fkey_inv(uint32_t k) {
    uint32_t u = (k >> 31) ? (k & 0x7fffffffu) : ~k;
    return __uint_as_float(u);
}

// ------------------------------------------------------------ shared types

// Per-tile statistics written by the indexer (or by the selection's own stats
// pass) for each run of TILE consecutive slots of one query.
constexpr int TILE = 256;
struct TileStat {
    float kmax2;     // max squared key norm over scored entries (0 if n/a)
    float smin;      // min finite score (+inf if none)
    float smax;      // max finite score (-inf if none)
    uint32_t nvalid; // number of finite scores
};

// Error-bound constant: |fp32 score - binary64 score| <= E with
//   E = 2^-22 (dI + HI + 2) * max_j ||k_j|| * sum_h |w_h| ||q_h||  (+ tiny)
// (each fp32 accumulation step is charged a relative error of 2^-22, twice the
// worst rounding of a truncating adder; see the indexer kernels).
__host__ __device__ inline double score_bound(double kmax, double sumwq, int HI, int dI) {
    return ldexp(1.0, -22) * double(dI + HI + 2) * kmax * sumwq * (1.0 + ldexp(1.0, -20)) + ldexp(1.0, -100);
}

// Scores ranked rounded to bfloat16 ("读完这篇，你就搞懂 DeepSeek v4 了", the
// passage on FP4 quantization-aware training: the indexer's score is
// quantized only down to BF16).  The rounded key r of an exact score x obeys
// |r - x| <= 2^-8 |x| + 2^-134 (half a spacing: 2^(e-8) in the binade
// [2^e, 2^(e+1)), 2^-134 among the subnormals) until x rounds past the
// largest finite value.  With |fp32 score - x| <= E and |fp32 score| <= M,
// the selection's bound for the keys is E plus this slack (slightly
// enlarged for the binary64 arithmetic); infinite when a key could overflow.
__host__ __device__ inline double bf16_key_bound(double E, double M) {
    const double x = M + E;
    if (!(x < 0x1.fe0p127)) return __builtin_inf();
    return E + (ldexp(1.0, -8) * x + ldexp(1.0, -134)) * (1.0 + ldexp(1.0, -40));
}

// A binary64 value rounded once to bfloat16, nearest with ties to even, as a
// binary64: in the normal range by rounding the 52-bit fraction to its top 7
// bits on the bit pattern (a carry may step the exponent; past 2^128 the
// result is infinite), below 2^-126 on a fixed spacing of 2^-133.  Zero,
// infinities and NaN pass through.
__device__ inline double bf16_round_key(double x) {
    const uint64_t u = (uint64_t)__double_as_longlong(x);
    const uint64_t mag = u & 0x7fffffffffffffffull, sign = u & 0x8000000000000000ull;
    const int ex = (int)(mag >> 52) - 1023;
    if (mag == 0 || ex == 1024) return x;
    if (ex >= -126) {
        const uint64_t keep = (mag >> 45) & 1u;
        uint64_t r = (mag + 0x00000fffffffffffull + keep) & ~0x00001fffffffffffull;
        if ((int)(r >> 52) - 1023 >= 128) r = 0x7ff0000000000000ull;
        return __longlong_as_double((long long)(r | sign));
    }
    const double r = rint(__longlong_as_double((long long)mag) * 0x1p133) * 0x1p-133;
    return __longlong_as_double((long long)((uint64_t)__double_as_longlong(r) | sign));
}

// sum_h |w_h| ||q_h|| in binary64 with a fixed reduction order: groups of 16
// threads take heads g, g + NT/16, ...; the 16 threads of a group split the
// head's row into 16 runs (one 16-byte load each when the row allows), square
// and sum them, and the group folds its 16 partial sums by a fixed tree.
template <int NT>
__device__ inline double block_sumwq(const void *qI, int dt, const float *w, int HI, int dI, int bq, double *dred) {
    const int g = threadIdx.x >> 4, r = threadIdx.x & 15;
    const int esz = dt == CSA2_F32 ? 4 : 2;
    const bool vec = (dI * esz == 256) && ((reinterpret_cast<uintptr_t>(qI) & 15) == 0);
    double acc = 0.0;
    for (int h = g; h < HI; h += NT / 16) {
        const size_t row = ((size_t)bq * HI + h) * dI;
        double q2 = 0.0;
        if (vec) {
            const u32x4 v = reinterpret_cast<const u32x4 *>(static_cast<const char *>(qI) + row * esz)[r];
#pragma unroll
            for (int e = 0; e < 4; e++) {
                if (dt == CSA2_F32) {
                    const double x = (double)__uint_as_float(v[e]);
                    q2 = fma(x, x, q2);
                } else {
                    const double x0 = (double)bf16_to_f32((uint16_t)(v[e] & 0xffffu));
                    const double x1 = (double)bf16_to_f32((uint16_t)(v[e] >> 16));
                    q2 = fma(x0, x0, q2);
                    q2 = fma(x1, x1, q2);
                }
            }
        } else {
            for (int d = r; d < dI; d += 16) {
                const double x = dt == CSA2_F32 ? (double)static_cast<const float *>(qI)[row + d]
                                                : (double)bf16_to_f32(static_cast<const uint16_t *>(qI)[row + d]);
                q2 = fma(x, x, q2);
            }
        }
        for (int o = 8; o > 0; o >>= 1) q2 += __shfl_xor(q2, o, 16);
        acc += fabs((double)w[(size_t)bq * HI + h]) * sqrt(q2);
    }
    if (r == 0) dred[g] = acc;
    __syncthreads();
    double t = 0.0;
    for (int i = 0; i < NT / 16; i++) t += dred[i];
    __syncthreads();
    return t;
}

}  // namespace csa2
