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
// bf16 rows of 128 or 512 channels: one matrix-core kernel that projects and
// pools (below).  Otherwise two kernels: the projection Z = X wz for every
// token row (a tiled fp32 GEMM from LDS), then the windowed per-channel
// softmax pooling, one thread per (entry, channel), reading Z and X once per
// window position.
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

// ---------------------------------------------------- bf16: matrix cores
// For bf16 rows the projection runs on the matrix cores and the pooling is
// fused behind it, so Z never goes through memory.  Block = EPB = 64 / m
// consecutive entries x 128 channels (eight waves); it needs the token rows
// of their windows, first(e0) .. first(e0) + (EPB + 1) m - 1 (at most 80),
// copied once into LDS (zero rows outside the context), and computes Z for
// those 80 rows: wave w takes channels c0 + 16 w .. + 15, its W^T fragments
// for all D held in registers (from a transposed copy of W), the 5 row
// tiles' X fragments read from LDS per 32-deep step.  Each Z element is one
// matrix-core dot product over d in a fixed order, whatever the block, so an
// entry comes out bitwise the same from a chunk with a halo as from the
// whole context.  Z goes to LDS; then each thread pools entries for its
// channel as the fp32 kernel does, the window's values read from the staged
// rows.
constexpr int CZ_ROWS = 80;  // 5 tiles of 16 rows: EPB m + m <= 64 + 16
constexpr int CZ_CH = 128;   // channels of a block
constexpr int CZ_NT = 64 * (CZ_CH / 16);

__global__ __launch_bounds__(256) void k_transpose_bf16(const uint16_t *__restrict__ w, int D,
                                                        uint16_t *__restrict__ wt) {
    __shared__ uint16_t t[32][33];
    const int bx = blockIdx.x * 32, by = blockIdx.y * 32;
    const int tx = threadIdx.x & 31, ty = threadIdx.x >> 5;
    for (int r = ty; r < 32; r += 8)
        if (by + r < D && bx + tx < D) t[r][tx] = w[(size_t)(by + r) * D + bx + tx];
    __syncthreads();
    for (int r = ty; r < 32; r += 8)
        if (bx + r < D && by + tx < D) wt[(size_t)(bx + r) * D + by + tx] = t[tx][r];
}

template <int D>
__global__ __launch_bounds__(CZ_NT) void k_compress_mfma(const uint16_t *__restrict__ x, const uint16_t *__restrict__ wt,
                                                         const float *__restrict__ bias, int64_t rows, int64_t n_out,
                                                         int m, int halo, uint16_t *__restrict__ out) {
    constexpr int KS = D / 32;
    constexpr int RT = CZ_ROWS / 16;
    constexpr int XS = D + 8;       // LDS stride of a staged row (16-bit elements)
    constexpr int ZS = CZ_CH + 1;
    constexpr int PPR = D / 8;      // 16-byte pieces of a row
    constexpr int XP = CZ_ROWS * PPR, XPT = (XP + CZ_NT - 1) / CZ_NT;
    __shared__ __attribute__((aligned(16))) uint16_t xs[CZ_ROWS * XS];
    __shared__ float zs[CZ_ROWS * ZS];
    const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
    const int col = lane & 15, kg = lane >> 4;
    const int epb = 64 / m;
    const int64_t e0 = (int64_t)blockIdx.y * epb;
    const int c0 = blockIdx.x * CZ_CH;
    const int64_t r0 = halo ? e0 * m : (e0 - 1) * m;  // token row of window position 0 of entry e0
    // the window rows, 16 bytes a thread per round (rows outside the context are zero)
    {
        const u32x4 zero = {0u, 0u, 0u, 0u};
        u32x4 v[XPT];
#pragma unroll
        for (int i = 0; i < XPT; i++) {
            const int pc = tid + CZ_NT * i;
            const int lr = pc / PPR, cc = pc % PPR;
            const int64_t r = r0 + lr;
            v[i] = (pc < XP && r >= 0 && r < rows) ? *reinterpret_cast<const u32x4 *>(x + (size_t)r * D + 8 * cc) : zero;
        }
#pragma unroll
        for (int i = 0; i < XPT; i++) {
            const int pc = tid + CZ_NT * i;
            if (pc < XP) *reinterpret_cast<u32x4 *>(xs + (pc / PPR) * XS + (pc % PPR) * 8) = v[i];
        }
    }
    // W^T fragments of this wave's 16 channels: B[d][c] = W[d][c] = Wt[c][d]
    u32x4 bw[KS];
    {
        const uint16_t *wr = wt + (size_t)(c0 + 16 * wave + col) * D + 8 * kg;
#pragma unroll
        for (int s2 = 0; s2 < KS; s2++) bw[s2] = *reinterpret_cast<const u32x4 *>(wr + 32 * s2);
    }
    __syncthreads();
    f32x4 acc[RT];
#pragma unroll
    for (int rt = 0; rt < RT; rt++) acc[rt] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int s2 = 0; s2 < KS; s2++) {
        u32x4 a[RT];
#pragma unroll
        for (int rt = 0; rt < RT; rt++) a[rt] = *reinterpret_cast<const u32x4 *>(xs + (16 * rt + col) * XS + 32 * s2 + 8 * kg);
#pragma unroll
        for (int rt = 0; rt < RT; rt++)
            acc[rt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, a[rt]),
                                                             __builtin_bit_cast(bf16x8, bw[s2]), acc[rt], 0, 0, 0);
    }
    // Z[row 16 rt + 4 kg + i][channel 16 wave + col] -> LDS
#pragma unroll
    for (int rt = 0; rt < RT; rt++)
#pragma unroll
        for (int i = 0; i < 4; i++) zs[(16 * rt + 4 * kg + i) * ZS + 16 * wave + col] = acc[rt][i];
    __syncthreads();
    // pooling: thread -> channel c0 + (tid % CZ_CH), entries e0 + tid / CZ_CH + (CZ_NT / CZ_CH) j
    const int cl = tid % CZ_CH, c = c0 + cl;
    for (int el = tid / CZ_CH; el < epb; el += CZ_NT / CZ_CH) {
        const int64_t i = e0 + el;
        if (i >= n_out) break;
        const int lr0 = el * m;  // local row of window position 0 (rows from r0)
        float l[32];
        float mx = -__builtin_inff();
        for (int r = 0; r < 2 * m; r++) {
            const int64_t t = r0 + lr0 + r;
            l[r] = -__builtin_inff();
            if (t < 0) continue;
            l[r] = zs[(lr0 + r) * ZS + cl] + bias[(size_t)r * D + c];
            mx = fmaxf(mx, l[r]);
        }
        float den = 0.f, a = 0.f;
        for (int r = 0; r < 2 * m; r++) {
            const int64_t t = r0 + lr0 + r;
            if (t < 0) continue;
            const float p = expf(l[r] - mx);
            den += p;
            a = fmaf(p, bf16_to_f32(xs[(lr0 + r) * XS + c]), a);
        }
        out[(size_t)i * D + c] = f32_to_bf16_rne(a / den);
    }
}

}  // namespace

static bool compress_mfma(int dt, int D) { return dt == CSA2_BF16 && (D == 128 || D == 512); }

size_t compress_workspace(int dt, int64_t n_out, int D, int m, int halo) {
    const int64_t rows = halo ? (n_out + 1) * m : n_out * m;
    Carve c(nullptr, 0);
    if (compress_mfma(dt, D)) c.take<uint16_t>((size_t)D * D);  // W^T
    else c.take<float>((size_t)rows * D);
    return c.used;
}

void compress_run(const void *x, int dt, int64_t n_out, int D, int m, int halo, const void *wz, const float *bias,
                  void *out, void *ws, size_t ws_bytes, hipStream_t s) {
    const int64_t rows = halo ? (n_out + 1) * m : n_out * m;
    Carve c(ws, ws_bytes);
    if (compress_mfma(dt, D)) {
        uint16_t *wt = c.take<uint16_t>((size_t)D * D);
        if (c.used > ws_bytes) throw Error(CSA2_EWORKSPACE, "compression workspace too small");
        hipLaunchKernelGGL(k_transpose_bf16, dim3((D + 31) / 32, (D + 31) / 32), dim3(256), 0, s,
                           static_cast<const uint16_t *>(wz), D, wt);
        check_launch("compression weights transpose");
        const int epb = 64 / m;
        const dim3 g(D / CZ_CH, (unsigned)((n_out + epb - 1) / epb));
        if (D == 512)
            hipLaunchKernelGGL(k_compress_mfma<512>, g, dim3(CZ_NT), 0, s, static_cast<const uint16_t *>(x), wt, bias,
                               rows, n_out, m, halo, static_cast<uint16_t *>(out));
        else
            hipLaunchKernelGGL(k_compress_mfma<128>, g, dim3(CZ_NT), 0, s, static_cast<const uint16_t *>(x), wt, bias,
                               rows, n_out, m, halo, static_cast<uint16_t *>(out));
        check_launch("compression (matrix cores)");
        return;
    }
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
