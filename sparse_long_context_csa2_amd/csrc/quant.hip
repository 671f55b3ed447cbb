// quant.hip -- FP4 quantizer for main-KV cache writes.
//
// "Recall之王 祭出Reuse", section "把KV Cache压到极致的几把杀手锏": the main KV
// is stored as E2M1 values with one E4M3 scale per 16 channels.  The pages
// give no recipe for choosing them; the reading taken, per 16-channel group:
// the scale is the smallest non-negative E4M3 value s with 6 s >= the group's
// largest magnitude (448 when none is), and each code is the E2M1 value
// nearest to x / s, ties to the even code, a zero stored as +0.
//
// No division is needed and every decision is exact in fp32: 6 s and the
// code boundaries (midpoint * s, midpoints 0.25 .. 5) have at most seven
// significant bits, so comparing them with |x| (a bf16 or fp32 value) is the
// exact comparison with the real quotient.
#include "internal.h"

namespace csa2 {
namespace {

// Value of a non-negative E4M3 ("FN") byte 0x00 .. 0x7E.
__device__ __forceinline__ float e4m3_pos(uint32_t b) {
    const uint32_t e = b >> 3, m = b & 7u;
    return e == 0 ? (float)m * 0x1p-9f : (float)(8u + m) * __builtin_ldexpf(1.f, (int)e - 10);
}

// One thread per 16-channel group of one row: 16 loads' worth of values, the
// scale by a 7-step search over the increasing positive bytes, the codes by
// counting the boundaries below |x| (a boundary tie goes to the even code:
// up across the boundaries after codes 1, 3 and 5).
template <bool F32>
__global__ __launch_bounds__(256) void k_quantize_fp4(const void *__restrict__ x, int64_t n, int D,
                                                      uint8_t *__restrict__ cache, const int64_t *__restrict__ dst_row) {
    const int gpr = D / 16;
    const int64_t t = (int64_t)blockIdx.x * 256 + threadIdx.x;
    const int64_t r = t / gpr;
    if (r >= n) return;
    const int g = (int)(t - r * gpr);
    float v[16];
    if constexpr (F32) {
        const f32x4 *p = reinterpret_cast<const f32x4 *>(static_cast<const float *>(x) + r * D + 16 * g);
#pragma unroll
        for (int u = 0; u < 4; u++) {
            const f32x4 q = p[u];
#pragma unroll
            for (int i = 0; i < 4; i++) v[4 * u + i] = q[i];
        }
    } else {
        const uint4 *p = reinterpret_cast<const uint4 *>(static_cast<const uint16_t *>(x) + r * D + 16 * g);
#pragma unroll
        for (int u = 0; u < 2; u++) {
            const uint4 q = p[u];
            const uint32_t w[4] = {q.x, q.y, q.z, q.w};
#pragma unroll
            for (int i = 0; i < 4; i++) {
                v[8 * u + 2 * i] = __uint_as_float(w[i] << 16);
                v[8 * u + 2 * i + 1] = __uint_as_float(w[i] & 0xffff0000u);
            }
        }
    }
    float amax = 0.f;
#pragma unroll
    for (int i = 0; i < 16; i++) amax = fmaxf(amax, fabsf(v[i]));
    // smallest byte b in [0, 0x7E] with 6 e4m3(b) >= amax, else 0x7E
    uint32_t lo = 0, hi = 0x7E;
    if (6.f * e4m3_pos(0x7E) >= amax) {
        while (lo < hi) {
            const uint32_t mid = (lo + hi) >> 1;
            if (6.f * e4m3_pos(mid) >= amax) hi = mid;
            else lo = mid + 1;
        }
    } else {
        lo = 0x7E;
    }
    const float s = e4m3_pos(lo);
    const float b0 = 0.25f * s, b1 = 0.75f * s, b2 = 1.25f * s, b3 = 1.75f * s, b4 = 2.5f * s, b5 = 3.5f * s,
                b6 = 5.f * s;
    uint32_t code[16];
#pragma unroll
    for (int i = 0; i < 16; i++) {
        const float a = fabsf(v[i]);
        uint32_t c = (uint32_t)(a > b0) + (uint32_t)(a >= b1) + (uint32_t)(a > b2) + (uint32_t)(a >= b3) +
                     (uint32_t)(a > b4) + (uint32_t)(a >= b5) + (uint32_t)(a > b6);
        if (s == 0.f) c = 0;
        code[i] = (v[i] < 0.f && c != 0) ? (c | 8u) : c;
    }
    uint32_t lo4 = 0, hi4 = 0;
#pragma unroll
    for (int i = 0; i < 8; i++) {
        const uint32_t byte = code[2 * i] | (code[2 * i + 1] << 4);
        if (i < 4) lo4 |= byte << (8 * i);
        else hi4 |= byte << (8 * (i - 4));
    }
    const int64_t row = dst_row ? dst_row[r] : r;
    uint8_t *dst = cache + row * (int64_t)(D / 2 + D / 16);
    uint8_t *cd = dst + 8 * g;
    if ((reinterpret_cast<uintptr_t>(cd) & 7u) == 0) {
        *reinterpret_cast<uint2 *>(cd) = make_uint2(lo4, hi4);
    } else {
#pragma unroll
        for (int i = 0; i < 4; i++) {
            cd[i] = (uint8_t)(lo4 >> (8 * i));
            cd[4 + i] = (uint8_t)(hi4 >> (8 * i));
        }
    }
    dst[D / 2 + g] = (uint8_t)lo;
}

}  // namespace

void launch_quantize_fp4(const void *x, int dt, int64_t n, int D, uint8_t *cache, const int64_t *dst_row,
                         hipStream_t s) {
    const int64_t threads = n * (D / 16);
    const dim3 grid((unsigned)((threads + 255) / 256));
    if (dt == CSA2_F32) hipLaunchKernelGGL(k_quantize_fp4<true>, grid, dim3(256), 0, s, x, n, D, cache, dst_row);
    else hipLaunchKernelGGL(k_quantize_fp4<false>, grid, dim3(256), 0, s, x, n, D, cache, dst_row);
    check_launch("FP4 quantize");
}

}  // namespace csa2
