// swa.hip -- the sliding-window (SWA) branch next to CSA2 and the merge of the
// two branches.
//
// Video transcript on V4.1 Flash (prism.simon-ai.net), passages on the SWA
// branch: every layer keeps its own uncompressed KV of the most recent 128
// tokens, never shared across layers, beside the shared global (CSA2) KV.
// Readings taken where the pages are silent:
//  - the window of a query at token position p is p - W + 1 .. p (its own
//    token the newest), rows of the same form as the global KV (one vector per
//    token, used as key and value by every head);
//  - the branches combine as one softmax over the union of their entries:
//    each branch's output weighted by its share exp(lse) of the joint
//    denominator.
// The window attention itself runs on the gather + attention kernels of the
// CSA2 branch (k = W entries, one split when W <= 128).
#include "internal.h"

namespace csa2 {
namespace {

constexpr float NEG_INF = -__builtin_inff();

// idx[bq][i] = p - W + 1 + i for the query's position p, or -1 where that is
// below 0 or at/after T (a position past the cache has no row).
__global__ __launch_bounds__(256) void k_window_idx(const int64_t *__restrict__ q_pos, int64_t BQ, int W, int64_t T,
                                                    int32_t *__restrict__ idx) {
    const int64_t g = (int64_t)blockIdx.x * 256 + threadIdx.x;
    if (g >= BQ * W) return;
    const int64_t bq = g / W;
    const int i = (int)(g - bq * W);
    const int64_t j = q_pos[bq] - W + 1 + i;
    idx[g] = (j < 0 || j >= T) ? -1 : (int32_t)j;
}

// One thread per 8 channels of one (query, head) row.  M = max(la, lb),
// u = e^(la - M), v = e^(lb - M): out = (u oa + v ob) / (u + v) and
// lse = M + ln(u + v); an empty branch (lse = -inf) has weight 0, both empty
// give 0 and -inf.  out may alias either input (each thread reads its own
// elements before writing them).
template <bool F32>
__global__ __launch_bounds__(256) void k_merge_attn(const void *oa_, const float *__restrict__ la_, const void *ob_,
                                                    const float *__restrict__ lb_, int64_t R, int D, void *out_,
                                                    float *lse) {
    const int tpr = D / 8;
    const int64_t g = (int64_t)blockIdx.x * 256 + threadIdx.x;
    const int64_t r = g / tpr;
    if (r >= R) return;
    const int c8 = (int)(g - r * tpr);
    const float la = la_[r], lb = lb_[r];
    const float M = fmaxf(la, lb);
    float u = 0.f, v = 0.f;
    if (M != NEG_INF) {
        u = __expf(la - M);  // exp(-inf) = 0
        v = __expf(lb - M);
    }
    const float s = u + v;
    const float inv = s > 0.f ? 1.f / s : 0.f;
    const float wu = u * inv, wv = v * inv;
    const size_t off = (size_t)r * D + 8 * c8;
    float a[8], b[8];
    if constexpr (F32) {
        const f32x4 *pa = reinterpret_cast<const f32x4 *>(static_cast<const float *>(oa_) + off);
        const f32x4 *pb = reinterpret_cast<const f32x4 *>(static_cast<const float *>(ob_) + off);
        const f32x4 a0 = pa[0], a1 = pa[1], b0 = pb[0], b1 = pb[1];
#pragma unroll
        for (int i = 0; i < 4; i++) {
            a[i] = a0[i];
            a[4 + i] = a1[i];
            b[i] = b0[i];
            b[4 + i] = b1[i];
        }
    } else {
        const uint4 pa = *reinterpret_cast<const uint4 *>(static_cast<const uint16_t *>(oa_) + off);
        const uint4 pb = *reinterpret_cast<const uint4 *>(static_cast<const uint16_t *>(ob_) + off);
        const uint32_t wa[4] = {pa.x, pa.y, pa.z, pa.w}, wb[4] = {pb.x, pb.y, pb.z, pb.w};
#pragma unroll
        for (int i = 0; i < 4; i++) {
            a[2 * i] = __uint_as_float(wa[i] << 16);
            a[2 * i + 1] = __uint_as_float(wa[i] & 0xffff0000u);
            b[2 * i] = __uint_as_float(wb[i] << 16);
            b[2 * i + 1] = __uint_as_float(wb[i] & 0xffff0000u);
        }
    }
    float o[8];
#pragma unroll
    for (int i = 0; i < 8; i++) o[i] = wu * a[i] + wv * b[i];
    if constexpr (F32) {
        f32x4 *po = reinterpret_cast<f32x4 *>(static_cast<float *>(out_) + off);
        po[0] = f32x4{o[0], o[1], o[2], o[3]};
        po[1] = f32x4{o[4], o[5], o[6], o[7]};
    } else {
        uint4 w;
        w.x = uint32_t(f32_to_bf16_rne(o[0])) | (uint32_t(f32_to_bf16_rne(o[1])) << 16);
        w.y = uint32_t(f32_to_bf16_rne(o[2])) | (uint32_t(f32_to_bf16_rne(o[3])) << 16);
        w.z = uint32_t(f32_to_bf16_rne(o[4])) | (uint32_t(f32_to_bf16_rne(o[5])) << 16);
        w.w = uint32_t(f32_to_bf16_rne(o[6])) | (uint32_t(f32_to_bf16_rne(o[7])) << 16);
        *reinterpret_cast<uint4 *>(static_cast<uint16_t *>(out_) + off) = w;
    }
    if (lse && c8 == 0) lse[r] = M == NEG_INF ? NEG_INF : M + __logf(s);
}

}  // namespace

void launch_window_idx(const int64_t *q_pos, int64_t BQ, int W, int64_t T, int32_t *idx, hipStream_t s) {
    const int64_t n = BQ * W;
    hipLaunchKernelGGL(k_window_idx, dim3((unsigned)((n + 255) / 256)), dim3(256), 0, s, q_pos, BQ, W, T, idx);
    check_launch("window list");
}

void launch_merge_attn(int dt, const void *oa, const float *la, const void *ob, const float *lb, int64_t R, int D,
                       void *out, float *lse, hipStream_t s) {
    const int64_t n = R * (D / 8);
    const dim3 grid((unsigned)((n + 255) / 256));
    if (dt == CSA2_F32) hipLaunchKernelGGL(k_merge_attn<true>, grid, dim3(256), 0, s, oa, la, ob, lb, R, D, out, lse);
    else hipLaunchKernelGGL(k_merge_attn<false>, grid, dim3(256), 0, s, oa, la, ob, lb, R, D, out, lse);
    check_launch("attention merge");
}

}  // namespace csa2
