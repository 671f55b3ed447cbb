// Gather + FP4 decode + shared-KV sparse attention for gfx950.
//
// "读完这篇，你就搞懂 DeepSeek v4 了", section "注意力计算（对应步骤三）", eq. (9):
// standard softmax attention in which the k entries chosen by the indexer form
// one matrix C, used as both keys and values by every query head:
//     a_j = scale * q_h . C_j,   o_h = sum_j softmax(a)_j C_j.
// "Recall之王 祭出Reuse", section "把KV Cache压到极致的几把杀手锏": the main KV
// may be stored as FP4 E2M1 with one E4M3 scale per 16 channels; the decoded
// value e2m1 * e4m3 has at most 5 significant bits and is exact in bf16.
//
// Matrix-core kernel: a block serves 16 heads of one query over a fixed split
// of 512 selected entries (the split depends only on k, so a query's result
// does not depend on the batch).  Each wave takes 32-entry sub-tiles: the
// gathered rows are staged in LDS as bf16 (FP4 rows decoded on the way in,
// to fp16, where they are also exact), S^T = C Q^T runs on the 16x16x32
// matrix-core instruction of that type with the rows as the A
// operand, the online softmax keeps one running max per head, and
// O^T = C^T P^T reuses the same LDS rows (read transposed) with P^T taken
// straight from the S^T result registers.  Waves merge through LDS; splits are
// merged by a small combine kernel.  Blocks of one (query, split) are placed
// on one XCD so the head groups share the gathered rows in L2.
#include "internal.h"

namespace csa2 {

constexpr int ATT_SPLIT = 512;  // selected entries per block (fixed)
constexpr int ATT_SUB = 32;     // entries per wave iteration

namespace {

constexpr float NEG_INF = -__builtin_inff();

// 4-bit E2M1 code -> binary32 bits (OCP MX element: bias 1, code 0bS001 = 0.5).
__device__ __forceinline__ uint32_t e2m1_bits(uint32_t c) {
    const uint32_t e = (c >> 1) & 3u, mb = c & 1u;
    const uint32_t mag = e ? (((e + 126u) << 23) | (mb << 22)) : (mb ? 0x3f000000u : 0u);
    return mag | ((c & 8u) << 28);
}
// E4M3 ("FN") byte -> float (bias 7; exponent field 0 is m * 2^-9).
__device__ __forceinline__ float e4m3_val(uint32_t s) {
    const uint32_t e = (s >> 3) & 15u, mt = s & 7u;
    const float mag = e ? __uint_as_float(((e + 120u) << 23) | (mt << 20)) : (float)mt * 0.001953125f;
    return (s & 0x80u) ? -mag : mag;
}
// Eight channels (one 32-bit code word, channel 2i in the low nibble of byte
// i) times one scale -> four packed bf16 pairs.  The products are exact in
// bf16, so dropping the low 16 bits of the fp32 product loses nothing.
__device__ __forceinline__ u32x4 fp4_dequant8(uint32_t word, float sc) {
    u32x4 r;
#pragma unroll
    for (int p = 0; p < 4; p++) {
        const uint32_t byte = (word >> (8 * p)) & 0xffu;
        const float v0 = __uint_as_float(e2m1_bits(byte & 15u)) * sc;
        const float v1 = __uint_as_float(e2m1_bits(byte >> 4)) * sc;
        r[p] = (__float_as_uint(v0) >> 16) | (__float_as_uint(v1) & 0xffff0000u);
    }
    return r;
}

// Same, packed as fp16 pairs: the products (<= 5 significant bits, magnitude
// in [2^-10, 2688]) are exact fp16 normals, so the conversion is exact.
__device__ __forceinline__ u32x4 fp4_dequant8_f16(uint32_t word, float sc) {
    u32x4 r;
#pragma unroll
    for (int p = 0; p < 4; p++) {
        const uint32_t byte = (word >> (8 * p)) & 0xffu;
        const float v0 = __uint_as_float(e2m1_bits(byte & 15u)) * sc;
        const float v1 = __uint_as_float(e2m1_bits(byte >> 4)) * sc;
        r[p] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_pkrtz(v0, v1));
    }
    return r;
}

__device__ __forceinline__ uint32_t pack_f16_rne(float a, float b) {
    const _Float16 ha = (_Float16)a, hb = (_Float16)b;
    return uint32_t(__builtin_bit_cast(uint16_t, ha)) | (uint32_t(__builtin_bit_cast(uint16_t, hb)) << 16);
}

// One 16x16x32 matrix-core step in the operand type of the staged rows:
// bf16 for bf16 KV, fp16 for FP4 KV (decoded FP4 values are exact in both;
// fp16 keeps three more bits of the softmax weights).
template <int FMT>
__device__ __forceinline__ f32x4 mma(u32x4 a, u32x4 b, f32x4 c) {
    if constexpr (FMT == CSA2_FP4)
        return __builtin_amdgcn_mfma_f32_16x16x32_f16(__builtin_bit_cast(f16x8, a), __builtin_bit_cast(f16x8, b), c,
                                                      0, 0, 0);
    else
        return __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, a), __builtin_bit_cast(bf16x8, b),
                                                       c, 0, 0, 0);
}

__device__ __forceinline__ float kv_elem(const uint8_t *row, int fmt, int D, int d) {
    if (fmt == CSA2_F32) return reinterpret_cast<const float *>(row)[d];
    if (fmt == CSA2_BF16) return bf16_to_f32(reinterpret_cast<const uint16_t *>(row)[d]);
    const uint32_t code = (row[d >> 1] >> ((d & 1) * 4)) & 15u;
    return __uint_as_float(e2m1_bits(code)) * e4m3_val(row[D / 2 + d / 16]);
}

__device__ __forceinline__ int64_t row_bytes(int fmt, int D) {
    return fmt == CSA2_F32 ? 4 * (int64_t)D : (fmt == CSA2_BF16 ? 2 * (int64_t)D : (int64_t)D / 2 + D / 16);
}

__device__ __forceinline__ void wave_lds_sync() {
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
}

// ------------------------------------------------------------ MFMA kernel
template <int D, int FMT>
__global__ __launch_bounds__(256, 1) void k_attn_mfma(const uint16_t *__restrict__ q, const uint8_t *__restrict__ kv,
                                                      int Q, int H, int64_t N, const int32_t *__restrict__ idx, int k,
                                                      float scale, int nsplit, uint16_t *__restrict__ out,
                                                      float *__restrict__ lse, float *__restrict__ part_o,
                                                      float2 *__restrict__ part_ml) {
    constexpr int KS = D / 32;  // contraction steps of S
    constexpr int DT = D / 16;  // 16-wide d tiles of O
    constexpr int ROWB = FMT == CSA2_FP4 ? D / 2 + D / 16 : 2 * D;
    constexpr int LS = D + 8;  // LDS row stride in bf16 (16 B pad)
    __shared__ __attribute__((aligned(16))) uint16_t tile[4 * ATT_SUB * LS];
    __shared__ float m_sh[4][16], l_sh[4][16], M_h[16], L_h[16];

    const int HG = H / 16;
    const int id = blockIdx.x, nb = gridDim.x;
    const int L = (nb % 8 == 0) ? (id % 8) * (nb / 8) + id / 8 : id;
    const int hg = L % HG;
    const int unit = L / HG;
    const int split = unit % nsplit;
    const int bq = unit / nsplit;
    const int b = bq / Q;
    const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
    const int col = lane & 15, kg = lane >> 4;
    uint16_t *T = tile + wave * ATT_SUB * LS;
    const u32x4 zero = {0u, 0u, 0u, 0u};

    // Query heads hg*16 + col as the B operand of S^T = C Q^T.
    u32x4 qf[KS];
    const uint16_t *qrow = q + ((size_t)bq * H + hg * 16 + col) * D + 8 * kg;
#pragma unroll
    for (int s = 0; s < KS; s++) qf[s] = *reinterpret_cast<const u32x4 *>(qrow + 32 * s);
    float qscale = scale;
    if constexpr (FMT == CSA2_FP4) {
        // bf16 queries -> fp16 operands, pre-scaled by a power of two when their
        // magnitude would overflow fp16 (the scale moves into the logits).
        float amax = 0.f;
#pragma unroll
        for (int s = 0; s < KS; s++)
#pragma unroll
            for (int e = 0; e < 4; e++)
                amax = fmaxf(amax, fmaxf(fabsf(bf16_to_f32(qf[s][e] & 0xffffu)), fabsf(bf16_to_f32(qf[s][e] >> 16))));
        amax = wave_max(amax);
        int ex = 0;
        if (amax > 32768.f) ex = (int)ceilf(log2f(amax / 32768.f));
        const float down = ldexpf(1.f, -ex);
        qscale = ldexpf(scale, ex);
#pragma unroll
        for (int s = 0; s < KS; s++)
#pragma unroll
            for (int e = 0; e < 4; e++)
                qf[s][e] = pack_f16_rne(bf16_to_f32(qf[s][e] & 0xffffu) * down, bf16_to_f32(qf[s][e] >> 16) * down);
    }

    f32x4 o[DT];
#pragma unroll
    for (int t = 0; t < DT; t++) o[t] = f32x4{0.f, 0.f, 0.f, 0.f};
    float m_run = NEG_INF, l_run = 0.f;

    const int e_begin = split * ATT_SPLIT;
    const int e_end = min(k, e_begin + ATT_SPLIT);
    const int32_t *irow = idx + (size_t)bq * k;
    const uint8_t *kvb = kv + (size_t)b * N * ROWB;

    for (int e0 = e_begin + wave * ATT_SUB; e0 < e_end; e0 += 4 * ATT_SUB) {
        const int my_e = e0 + (lane & 31);
        int jr = my_e < e_end ? irow[my_e] : -1;
        if (jr >= N) jr = -1;  // out-of-range entries are skipped like -1
        // ---- gather the 32 rows into LDS as bf16
        if constexpr (FMT == CSA2_BF16) {
            constexpr int CPR = D / 8;  // 16-byte chunks per row

            for (int c = lane; c < ATT_SUB * CPR; c += 64) {
                const int r = c / CPR, cc = c % CPR;
                const int j = __shfl(jr, r);
                u32x4 v = zero;
                if (j >= 0) v = *reinterpret_cast<const u32x4 *>(kvb + (size_t)j * ROWB + cc * 16);
                *reinterpret_cast<u32x4 *>(T + r * LS + cc * 8) = v;
            }
        } else {
            constexpr int CPR = D / 32;  // 16-byte code chunks (32 channels) per row

            for (int c = lane; c < ATT_SUB * CPR; c += 64) {
                const int r = c / CPR, cc = c % CPR;
                const int j = __shfl(jr, r);
                u32x4 codes = zero;
                uint32_t sc2 = 0;
                if (j >= 0) {
                    const uint8_t *row = kvb + (size_t)j * ROWB;
                    codes = *reinterpret_cast<const u32x4 *>(row + cc * 16);
                    sc2 = *reinterpret_cast<const uint16_t *>(row + D / 2 + cc * 2);
                }
                const float s0 = e4m3_val(sc2 & 0xffu), s1 = e4m3_val(sc2 >> 8);
                uint16_t *dst = T + r * LS + cc * 32;
                *reinterpret_cast<u32x4 *>(dst) = fp4_dequant8_f16(codes[0], s0);
                *reinterpret_cast<u32x4 *>(dst + 8) = fp4_dequant8_f16(codes[1], s0);
                *reinterpret_cast<u32x4 *>(dst + 16) = fp4_dequant8_f16(codes[2], s1);
                *reinterpret_cast<u32x4 *>(dst + 24) = fp4_dequant8_f16(codes[3], s1);
            }
        }
        wave_lds_sync();
        // ---- S^T[e][h] for the two 16-entry halves
        f32x4 st[2];
#pragma unroll
        for (int t = 0; t < 2; t++) {
            st[t] = f32x4{0.f, 0.f, 0.f, 0.f};
            const uint16_t *arow = T + (t * 16 + col) * LS + 8 * kg;
#pragma unroll
            for (int s = 0; s < KS; s++) {
                const u32x4 a = *reinterpret_cast<const u32x4 *>(arow + 32 * s);
                st[t] = mma<FMT>(a, qf[s], st[t]);
            }
        }
        // ---- online softmax for head col; this lane holds entries 16t + 4kg + i
        float a[8];
        float mt = NEG_INF;
#pragma unroll
        for (int t = 0; t < 2; t++)
#pragma unroll
            for (int i = 0; i < 4; i++) {
                const int j = __shfl(jr, t * 16 + 4 * kg + i);
                const float v = j >= 0 ? st[t][i] * qscale : NEG_INF;
                a[t * 4 + i] = v;
                mt = fmaxf(mt, v);
            }
        mt = fmaxf(mt, __shfl_xor(mt, 16));
        mt = fmaxf(mt, __shfl_xor(mt, 32));
        const float m_new = fmaxf(m_run, mt);
        const float alpha = m_run == NEG_INF ? 0.f : __expf(m_run - m_new);
        float psum = 0.f;
        uint32_t pk[4];
#pragma unroll
        for (int x = 0; x < 8; x += 2) {
            const float p0 = a[x] == NEG_INF ? 0.f : __expf(a[x] - m_new);
            const float p1 = a[x + 1] == NEG_INF ? 0.f : __expf(a[x + 1] - m_new);
            psum += p0 + p1;
            if constexpr (FMT == CSA2_FP4) pk[x / 2] = pack_f16_rne(p0, p1);
            else pk[x / 2] = uint32_t(f32_to_bf16_rne(p0)) | (uint32_t(f32_to_bf16_rne(p1)) << 16);
        }
        l_run = l_run * alpha + psum;
        m_run = m_new;
        const u32x4 pb = {pk[0], pk[1], pk[2], pk[3]};
        // ---- O^T[d][h] += C^T[d][e] P^T[e][h]; element x of the A operand is
        // row 16(x/4) + 4kg + x%4 of the staged tile, matching pb element x.
        const uint16_t *cb = T + (4 * kg) * LS + col;
#pragma unroll
        for (int t = 0; t < DT; t++) {
            uint32_t w4[4];
#pragma unroll
            for (int x = 0; x < 8; x += 2) {
                const int r0 = 16 * (x / 4) + (x % 4);
                w4[x / 2] = uint32_t(cb[r0 * LS + 16 * t]) | (uint32_t(cb[(r0 + 1) * LS + 16 * t]) << 16);
            }
            const u32x4 av = {w4[0], w4[1], w4[2], w4[3]};
            o[t] = o[t] * alpha;
            o[t] = mma<FMT>(av, pb, o[t]);
        }
        wave_lds_sync();
    }

    // ---- merge the four waves (same heads, disjoint entries)
    l_run += __shfl_xor(l_run, 16);
    l_run += __shfl_xor(l_run, 32);
    if (kg == 0) {
        m_sh[wave][col] = m_run;
        l_sh[wave][col] = l_run;
    }
    __syncthreads();
    float M = NEG_INF;
#pragma unroll
    for (int w = 0; w < 4; w++) M = fmaxf(M, m_sh[w][col]);
    float Ls = 0.f;
#pragma unroll
    for (int w = 0; w < 4; w++) Ls += m_sh[w][col] == NEG_INF ? 0.f : l_sh[w][col] * __expf(m_sh[w][col] - M);
    const float mine = m_run == NEG_INF ? 0.f : __expf(m_run - M);
    if (wave == 0 && kg == 0) {
        M_h[col] = M;
        L_h[col] = Ls;
    }
    float *ob = reinterpret_cast<float *>(tile);  // [16 heads][D]
    for (int w = 0; w < 4; w++) {
        if (wave == w) {
#pragma unroll
            for (int t = 0; t < DT; t++)
#pragma unroll
                for (int r = 0; r < 4; r++) {
                    const int i = col * D + 16 * t + 4 * kg + r;
                    const float v = o[t][r] * mine;
                    ob[i] = w == 0 ? v : ob[i] + v;
                }
        }
        __syncthreads();
    }
    if (nsplit == 1) {
        for (int i = threadIdx.x; i < 16 * D; i += 256) {
            const int h = i / D, d = i % D;
            const float Lh = L_h[h];
            const float v = Lh > 0.f ? ob[i] / Lh : 0.f;
            out[((size_t)bq * H + hg * 16 + h) * D + d] = f32_to_bf16_rne(v);
        }
        if (lse && threadIdx.x < 16) {
            const float Lh = L_h[threadIdx.x];
            lse[(size_t)bq * H + hg * 16 + threadIdx.x] = Lh > 0.f ? M_h[threadIdx.x] + logf(Lh) : NEG_INF;
        }
    } else {
        const size_t pbase = ((size_t)bq * nsplit + split) * H + hg * 16;
        for (int i = threadIdx.x; i < 16 * D; i += 256) part_o[pbase * D + i] = ob[i];
        if (threadIdx.x < 16) part_ml[pbase + threadIdx.x] = make_float2(M_h[threadIdx.x], L_h[threadIdx.x]);
    }
}

// ----------------------------------------------------------- split merge
__global__ __launch_bounds__(256) void k_attn_combine(const float *__restrict__ part_o,
                                                      const float2 *__restrict__ part_ml, int H, int D, int nsplit,
                                                      void *__restrict__ out, int out_dt, float *__restrict__ lse) {
    const int bq = blockIdx.y, h = blockIdx.x;
    float M = NEG_INF;
    for (int s = 0; s < nsplit; s++) M = fmaxf(M, part_ml[((size_t)bq * nsplit + s) * H + h].x);
    float Ls = 0.f;
    for (int s = 0; s < nsplit; s++) {
        const float2 ml = part_ml[((size_t)bq * nsplit + s) * H + h];
        Ls += ml.x == NEG_INF ? 0.f : ml.y * __expf(ml.x - M);
    }
    for (int d = threadIdx.x; d < D; d += 256) {
        float acc = 0.f;
        for (int s = 0; s < nsplit; s++) {
            const size_t pi = ((size_t)bq * nsplit + s) * H + h;
            const float mx = part_ml[pi].x;
            if (mx != NEG_INF) acc += part_o[pi * D + d] * __expf(mx - M);
        }
        const float v = Ls > 0.f ? acc / Ls : 0.f;
        const size_t oi = ((size_t)bq * H + h) * D + d;
        if (out_dt == CSA2_F32) static_cast<float *>(out)[oi] = v;
        else static_cast<uint16_t *>(out)[oi] = f32_to_bf16_rne(v);
    }
    if (lse && threadIdx.x == 0) lse[(size_t)bq * H + h] = Ls > 0.f ? M + logf(Ls) : NEG_INF;
}

// ------------------------------------------------------------ VALU kernel
// Any head count, dim and format: one block per (query, head), fp32 math.
__global__ __launch_bounds__(256) void k_attn_valu(const void *__restrict__ q, int q_dt,
                                                   const uint8_t *__restrict__ kv, int kv_dt, int Q, int H, int D,
                                                   int64_t N, const int32_t *__restrict__ idx, int k, float scale,
                                                   void *__restrict__ out, float *__restrict__ lse) {
    extern __shared__ float sh[];  // q row [D], logits [k]
    __shared__ float red[256];
    float *qs = sh, *as = sh + D;
    const int bq = blockIdx.y, h = blockIdx.x;
    const int b = bq / Q;
    const int64_t rb = row_bytes(kv_dt, D);
    const uint8_t *kvb = kv + (size_t)b * N * rb;
    const size_t qoff = ((size_t)bq * H + h) * D;
    for (int d = threadIdx.x; d < D; d += 256)
        qs[d] = q_dt == CSA2_F32 ? static_cast<const float *>(q)[qoff + d]
                                 : bf16_to_f32(static_cast<const uint16_t *>(q)[qoff + d]);
    __syncthreads();
    const int32_t *irow = idx + (size_t)bq * k;
    float mx = NEG_INF;
    for (int t = threadIdx.x; t < k; t += 256) {
        const int32_t j = irow[t];
        float a = NEG_INF;
        if (j >= 0 && j < N) {
            const uint8_t *row = kvb + (size_t)j * rb;
            float dot = 0.f;
            for (int d = 0; d < D; d++) dot = fmaf(qs[d], kv_elem(row, kv_dt, D, d), dot);
            a = scale * dot;
        }
        as[t] = a;
        mx = fmaxf(mx, a);
    }
    red[threadIdx.x] = mx;
    __syncthreads();
    for (int o = 128; o > 0; o >>= 1) {
        if (threadIdx.x < o) red[threadIdx.x] = fmaxf(red[threadIdx.x], red[threadIdx.x + o]);
        __syncthreads();
    }
    const float M = red[0];
    __syncthreads();
    float z = 0.f;
    for (int t = threadIdx.x; t < k; t += 256) {
        const float p = as[t] == NEG_INF ? 0.f : expf(as[t] - M);
        as[t] = p;
        z += p;
    }
    red[threadIdx.x] = z;
    __syncthreads();
    for (int o = 128; o > 0; o >>= 1) {
        if (threadIdx.x < o) red[threadIdx.x] += red[threadIdx.x + o];
        __syncthreads();
    }
    const float Z = red[0];
    for (int d = threadIdx.x; d < D; d += 256) {
        float acc = 0.f;
        for (int t = 0; t < k; t++) {
            const int32_t j = irow[t];
            if (j >= 0 && j < N && as[t] != 0.f) acc = fmaf(as[t], kv_elem(kvb + (size_t)j * rb, kv_dt, D, d), acc);
        }
        const float v = Z > 0.f ? acc / Z : 0.f;
        if (q_dt == CSA2_F32) static_cast<float *>(out)[qoff + d] = v;
        else static_cast<uint16_t *>(out)[qoff + d] = f32_to_bf16_rne(v);
    }
    if (lse && threadIdx.x == 0) lse[(size_t)bq * H + h] = Z > 0.f ? M + logf(Z) : NEG_INF;
}

template <int D, int FMT>
void launch_mfma(const AttnPlan &p, const void *q, const void *kv, const int32_t *idx, float scale, void *out,
                 float *lse, float *part_o, float2 *part_ml, hipStream_t s) {
    const int blocks = p.B * p.Q * p.nsplit * (p.H / 16);
    hipLaunchKernelGGL((k_attn_mfma<D, FMT>), dim3(blocks), dim3(256), 0, s, static_cast<const uint16_t *>(q),
                       static_cast<const uint8_t *>(kv), p.Q, p.H, p.N, idx, p.k, scale, p.nsplit,
                       static_cast<uint16_t *>(out), lse, part_o, part_ml);
}

}  // namespace

AttnPlan attn_plan(int q_dt, int kv_dt, int B, int Q, int H, int D, int64_t N, int k) {
    AttnPlan p{q_dt, kv_dt, B, Q, H, D, N, k, false, 1};
    p.mfma = q_dt == CSA2_BF16 && (kv_dt == CSA2_BF16 || kv_dt == CSA2_FP4) && H % 16 == 0 &&
             (D == 64 || D == 128 || D == 256 || D == 512);
    p.nsplit = p.mfma ? (k + ATT_SPLIT - 1) / ATT_SPLIT : 1;
    return p;
}

bool attn_supported(const AttnPlan &p) { return p.mfma || (p.D + p.k) <= 16384; }

size_t attn_workspace(const AttnPlan &p) {
    if (!p.mfma || p.nsplit == 1) return 0;
    Carve c(nullptr, 0);
    c.take<float>((size_t)p.B * p.Q * p.nsplit * p.H * p.D);
    c.take<float2>((size_t)p.B * p.Q * p.nsplit * p.H);
    return c.used;
}

void attn_run(const AttnPlan &p, const void *q, const void *kv, const int32_t *idx, float scale, void *out,
              float *lse, void *ws, size_t ws_bytes, hipStream_t s) {
    const int BQ = p.B * p.Q;
    if (!p.mfma) {
        size_t lds = sizeof(float) * ((size_t)p.D + p.k);
        hipLaunchKernelGGL(k_attn_valu, dim3(p.H, BQ), dim3(256), lds, s, q, p.q_dt,
                           static_cast<const uint8_t *>(kv), p.kv_dt, p.Q, p.H, p.D, p.N, idx, p.k, scale, out, lse);
        check_launch("attention (vector)");
        return;
    }
    float *part_o = nullptr;
    float2 *part_ml = nullptr;
    if (p.nsplit > 1) {
        Carve c(ws, ws_bytes);
        part_o = c.take<float>((size_t)BQ * p.nsplit * p.H * p.D);
        part_ml = c.take<float2>((size_t)BQ * p.nsplit * p.H);
        if (c.used > ws_bytes) throw Error(CSA2_EWORKSPACE, "attention workspace too small");
    }
#define CSA2_ATT_CASE(d)                                                                             \
    case d:                                                                                          \
        if (p.kv_dt == CSA2_FP4) launch_mfma<d, CSA2_FP4>(p, q, kv, idx, scale, out, lse, part_o, part_ml, s); \
        else launch_mfma<d, CSA2_BF16>(p, q, kv, idx, scale, out, lse, part_o, part_ml, s);                   \
        break;
    switch (p.D) {
        CSA2_ATT_CASE(64)
        CSA2_ATT_CASE(128)
        CSA2_ATT_CASE(256)
        CSA2_ATT_CASE(512)
    }
#undef CSA2_ATT_CASE
    check_launch("attention");
    if (p.nsplit > 1) {
        hipLaunchKernelGGL(k_attn_combine, dim3(p.H, BQ), dim3(256), 0, s, part_o, part_ml, p.H, p.D, p.nsplit, out,
                           p.q_dt, lse);
        check_launch("attention combine");
    }
}

}  // namespace csa2
