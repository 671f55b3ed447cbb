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
__device__ __forceinline__ float bf16_to_f32(uint16_t h) { return __uint_as_float(uint32_t(h) << 16); }

// Round-to-nearest-even fp32 -> bf16 bits (inputs are finite).
__device__ __forceinline__ uint16_t f32_to_bf16_rne(float f) {
    uint32_t u = __float_as_uint(f);
    u += 0x7fffu + ((u >> 16) & 1u);
    return uint16_t(u >> 16);
}

__device__ __forceinline__ float wave_sum(float v) {
    for (int o = 32; o > 0; o >>= 1) v += __shfl_xor(v, o);
    return v;
}
__device__ __forceinline__ float wave_max(float v) {
    for (int o = 32; o > 0; o >>= 1) v = fmaxf(v, __shfl_xor(v, o));
    return v;
}
__device__ __forceinline__ float wave_min(float v) {
    for (int o = 32; o > 0; o >>= 1) v = fminf(v, __shfl_xor(v, o));
    return v;
}
__device__ __forceinline__ uint32_t wave_sum_u32(uint32_t v) {
    for (int o = 32; o > 0; o >>= 1) v += __shfl_xor(v, o);
    return v;
}

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

}  // namespace csa2
