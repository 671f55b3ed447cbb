// Token compression for gfx950.
//
// "读完这篇，你就搞懂 DeepSeek v4 了": the HCA "压缩机制" paragraphs (eqs. 10, 11)
// describe CSA's compression by contrast -- groups of m tokens, two
// consecutive groups concatenated, weights S = softmax over a projection Z
// plus a learnable bias B, applied to the values.  Entry i pools window
// positions r = 0..2m-1 (previous group, then its own group), per channel c:
//     l_r[c] = x_t . wz[:, c] + bias[r][c],   out_i[c] = sum_r softmax_r(l[c]) x_t[c]
// Positions before token 0 are dropped.
//
// Two kernels: the projection Z = X wz for every token row (a tiled fp32 GEMM
// from LDS), then the windowed per-channel softmax pooling, one thread per
// (entry, channel), reading Z and X once per window position.
#include "internal.h"

namespace csa2 {
namespace {

__device__ __forceinline__ float ld(const void *p, int dt, size_t i) {
    return dt == CSA2_F32 ? static_cast<const float *>(p)[i] : bf16_to_f32(static_cast<const uint16_t *>(p)[i]);
}

// Z[rows, D] = X[rows, D] * W[D, D] (fp32 accumulate); 64x64 output tile per
// block, 16-deep k steps staged in LDS, 4x4 outputs per thread.
__global__ __launch_bounds__(256) void k_compress_z(const void *__restrict__ x, const void *__restrict__ wz, int dt,
                                                    int64_t rows, int D, float *__restrict__ Z) {
    __shared__ float As[16][65];
    __shared__ float Bs[16][65];
    const int64_t row0 = (int64_t)blockIdx.y * 64;
    const int col0 = blockIdx.x * 64;
    const int tid = threadIdx.x;
    const int tr = tid / 16, tc = tid % 16;
    float acc[4][4] = {};
    for (int k0 = 0; k0 < D; k0 += 16) {
        for (int i = 0; i < 4; i++) {
            const int e = tid * 4 + i;
            const int r = e / 16, kk = e % 16;
            As[kk][r] = row0 + r < rows ? ld(x, dt, (size_t)(row0 + r) * D + k0 + kk) : 0.f;
            const int kb = e / 64, c = e % 64;
            Bs[kb][c] = col0 + c < D ? ld(wz, dt, (size_t)(k0 + kb) * D + col0 + c) : 0.f;
        }
        __syncthreads();
#pragma unroll
        for (int kk = 0; kk < 16; kk++) {
            float a[4], b[4];
#pragma unroll
            for (int i = 0; i < 4; i++) {
                a[i] = As[kk][tr * 4 + i];
                b[i] = Bs[kk][tc * 4 + i];
            }
#pragma unroll
            for (int i = 0; i < 4; i++)
#pragma unroll
                for (int j = 0; j < 4; j++) acc[i][j] = fmaf(a[i], b[j], acc[i][j]);
        }
        __syncthreads();
    }
    for (int i = 0; i < 4; i++) {
        const int64_t r = row0 + tr * 4 + i;
        if (r >= rows) continue;
        for (int j = 0; j < 4; j++) {
            const int c = col0 + tc * 4 + j;
            if (c < D) Z[(size_t)r * D + c] = acc[i][j];
        }
    }
}

__global__ __launch_bounds__(256) void k_compress_pool(const void *__restrict__ x, int dt, const float *__restrict__ Z,
                                                       const float *__restrict__ bias, int64_t n_out, int D, int m,
                                                       int halo, void *__restrict__ out) {
    const int64_t e = (int64_t)blockIdx.x * 256 + threadIdx.x;
    const int64_t i = e / D;
    const int c = (int)(e % D);
    if (i >= n_out) return;
    const int64_t first = halo ? i * m : (i - 1) * m;  // x row of window position 0
    float l[32];
    float mx = -__builtin_inff();
    for (int r = 0; r < 2 * m; r++) {
        const int64_t t = first + r;
        l[r] = -__builtin_inff();
        if (t < 0) continue;
        l[r] = Z[(size_t)t * D + c] + bias[(size_t)r * D + c];
        mx = fmaxf(mx, l[r]);
    }
    float den = 0.f, acc = 0.f;
    for (int r = 0; r < 2 * m; r++) {
        const int64_t t = first + r;
        if (t < 0) continue;
        const float p = expf(l[r] - mx);
        den += p;
        acc = fmaf(p, ld(x, dt, (size_t)t * D + c), acc);
    }
    const float v = acc / den;
    if (dt == CSA2_F32) static_cast<float *>(out)[(size_t)i * D + c] = v;
    else static_cast<uint16_t *>(out)[(size_t)i * D + c] = f32_to_bf16_rne(v);
}

}  // namespace

size_t compress_workspace(int dt, int64_t n_out, int D, int m, int halo) {
    (void)dt;
    const int64_t rows = halo ? (n_out + 1) * m : n_out * m;
    Carve c(nullptr, 0);
    c.take<float>((size_t)rows * D);
    return c.used;
}

void compress_run(const void *x, int dt, int64_t n_out, int D, int m, int halo, const void *wz, const float *bias,
                  void *out, void *ws, size_t ws_bytes, hipStream_t s) {
    const int64_t rows = halo ? (n_out + 1) * m : n_out * m;
    Carve c(ws, ws_bytes);
    float *Z = c.take<float>((size_t)rows * D);
    if (c.used > ws_bytes) throw Error(CSA2_EWORKSPACE, "compression workspace too small");
    dim3 g1((D + 63) / 64, (unsigned)((rows + 63) / 64));
    hipLaunchKernelGGL(k_compress_z, g1, dim3(256), 0, s, x, wz, dt, rows, D, Z);
    check_launch("compression projection");
    const int64_t total = n_out * D;
    hipLaunchKernelGGL(k_compress_pool, dim3((unsigned)((total + 255) / 256)), dim3(256), 0, s, x, dt, Z, bias, n_out,
                       D, m, halo, out);
    check_launch("compression pooling");
}

}  // namespace csa2
