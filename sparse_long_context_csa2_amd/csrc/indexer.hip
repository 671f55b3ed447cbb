// Lightning-indexer score kernels for gfx950.
//
// "读完这篇，你就搞懂 DeepSeek v4 了", section "闪电索引机制（对应步骤二）", eq. (8):
// every compressed entry j is scored against the query token per indexer head,
// the head scores are weighted and summed -- with DSA's per-head ReLU:
//     s(j) = sum_h w_h * ReLU(q_h . k_j)
//
// Decode streams the whole key cache once per query (HBM-bound), but the
// 64-head contraction is 64 FLOP per key byte, above the fp32 VALU ridge, so
// the bf16 kernel runs it on the matrix cores: v_mfma_f32_16x16x32_bf16 with
// the query heads as the A operand (resident in registers for the block) and
// 16 key rows per B operand, loaded straight from HBM with 64-byte coalesced
// row segments.  The epilogue (ReLU, head weights, head sum) and the per-entry
// squared key norm used by the error bound are fused; each block also writes
// min/max/count statistics of its 256 scores for the selection that follows.
#include "internal.h"

namespace csa2 {

namespace {

constexpr float NEG_INF = -__builtin_inff();
constexpr float POS_INF = __builtin_inff();

__device__ __forceinline__ int64_t visible_entries(const int64_t *q_pos, int bq, int m, int64_t N) {
    if (!q_pos) return N;
    int64_t t = q_pos[bq];
    if (t < 0) return 0;
    int64_t v = (t + 1) / m;
    return v < N ? v : N;
}

// Block-wide reduction of per-thread tile statistics; thread 0 writes.
__device__ void reduce_tile_stat(float smin, float smax, uint32_t nval, float kmax2, TileStat *dst) {
    __shared__ float r_min[4], r_max[4], r_k[4];
    __shared__ uint32_t r_n[4];
    const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
    smin = wave_min(smin);
    smax = wave_max(smax);
    kmax2 = wave_max(kmax2);
    nval = wave_sum_u32(nval);
    if (lane == 0) {
        r_min[wave] = smin;
        r_max[wave] = smax;
        r_k[wave] = kmax2;
        r_n[wave] = nval;
    }
    __syncthreads();
    if (threadIdx.x == 0) {
        TileStat t;
        t.smin = fminf(fminf(r_min[0], r_min[1]), fminf(r_min[2], r_min[3]));
        t.smax = fmaxf(fmaxf(r_max[0], r_max[1]), fmaxf(r_max[2], r_max[3]));
        t.kmax2 = fmaxf(fmaxf(r_k[0], r_k[1]), fmaxf(r_k[2], r_k[3]));
        t.nvalid = r_n[0] + r_n[1] + r_n[2] + r_n[3];
        *dst = t;
    }
}

// --------------------------------------------------------------- MFMA path
// Block = 4 waves = 256 slots (one statistics tile); each wave scores 4
// groups of 16 slots.  MFMA operand layouts (16x16x32, wave64): lane l holds
// A[l%16][8*(l/16) .. +8] and B[8*(l/16) .. +8][l%16]; the result tile has
// D[4*(l/16) + r][l%16] in element r.  Both operands use the same lane ->
// k mapping, so every product pairs q[h][d] with k[j][d] for the same d.
// FP4 indexer keys (KFP4): rows of DI/2 code bytes and DI/16 E4M3 scale
// bytes; lane l loads the 4 code bytes of its 8 channels per contraction step
// and their scale byte, and decodes them to bf16 in registers (exact: at most
// 6 significant bits), so the matrix-core step and everything after it are
// the bf16 path's.
typedef float __attribute__((ext_vector_type(2))) idx_f32x2;
typedef __bf16 __attribute__((ext_vector_type(2))) idx_bf16x2;  // converted to with round-to-nearest-even

// ReLU of a matrix-core result as one integer maximum on its bits: a float
// whose sign bit is set is a negative integer, so max(bits, 0) keeps x >= +0
// and gives +0 for negatives (the float maximum would first canonicalize x
// for NaNs, a second instruction per value).
__device__ __forceinline__ float relu_bits(float x) { return __int_as_float(max(__float_as_int(x), 0)); }

template <int DI>
__device__ __forceinline__ u32x4 fp4_keys_to_bf16x8(uint32_t word, uint32_t sbyte) {
    // scale = pow2 * f: the conversion instruction applies the power of two,
    // an fp32 multiply the mantissa factor f = +-1.mmm (at most 4 significant
    // bits); every product is exact, and so is its bf16 rounding
    const uint32_t mag = e4m3_mag_bits(sbyte);
    const float pow2 = __uint_as_float(mag & 0x7f800000u);
    const float f = mag ? __uint_as_float((mag & 0x007fffffu) | 0x3f800000u | ((sbyte & 0x80u) << 24)) : 0.f;
    u32x4 r;
    idx_f32x2 v0 = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(word, pow2, 0);
    idx_f32x2 v1 = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(word, pow2, 1);
    idx_f32x2 v2 = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(word, pow2, 2);
    idx_f32x2 v3 = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(word, pow2, 3);
    r[0] = __builtin_bit_cast(uint32_t, __builtin_convertvector(v0 * f, idx_bf16x2));
    r[1] = __builtin_bit_cast(uint32_t, __builtin_convertvector(v1 * f, idx_bf16x2));
    r[2] = __builtin_bit_cast(uint32_t, __builtin_convertvector(v2 * f, idx_bf16x2));
    r[3] = __builtin_bit_cast(uint32_t, __builtin_convertvector(v3 * f, idx_bf16x2));
    return r;
}

template <int HI, int DI, bool KFP4>
__global__ __launch_bounds__(256, 2) void k_index_mfma(const uint16_t *__restrict__ qI, const float *__restrict__ w,
                                                       const uint16_t *__restrict__ kI, int Q, int64_t N,
                                                       const int64_t *__restrict__ q_pos, int m,
                                                       const int32_t *__restrict__ cand, int P,
                                                       float *__restrict__ scores, TileStat *__restrict__ stats,
                                                       int ntiles, double *__restrict__ sumwq) {
    constexpr int HT = HI / 16;  // head tiles
    constexpr int KS = DI / 32;  // contraction steps
    constexpr int G = 4;         // 16-slot groups per wave
    const int bq = blockIdx.y;
    const int b = bq / Q;
    const int tile = blockIdx.x;
    const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
    const int col = lane & 15, kg = lane >> 4;
    const int64_t n = cand ? (int64_t)P : N;
    const int64_t nvis = visible_entries(q_pos, bq, m, N);

    // Row indices of this wave's 4 x 16 slots.
    const int64_t slot0 = (int64_t)tile * TILE + wave * 64;
    int64_t jrow[G];
    bool valid[G];
#pragma unroll
    for (int g = 0; g < G; g++) {
        int64_t slot = slot0 + g * 16 + col;
        int64_t j = -1;
        if (slot < n) j = cand ? (int64_t)cand[(int64_t)bq * P + slot] : slot;
        valid[g] = (j >= 0) && (j < nvis);
        jrow[g] = valid[g] ? j : 0;
    }
    // Issue every key load of the wave first (64 B per lane per group; FP4:
    // 16 code bytes and 4 scale bytes, decoded after the query loads).
    u32x4 kb[G][KS];
    const u32x4 zero = {0u, 0u, 0u, 0u};
    uint32_t kw4[KFP4 ? G : 1][KS], ks4[KFP4 ? G : 1][KS];
#pragma unroll
    for (int g = 0; g < G; g++) {
        if constexpr (KFP4) {
            // lane group kg holds channels kg DI/4 .. + DI/4 - 1 (step s: + 8 s ..
            // + 8 s + 7): its DI/8 code bytes and DI/64 scale bytes are contiguous
            constexpr int RB = DI / 2 + DI / 16;
            const uint8_t *krow = reinterpret_cast<const uint8_t *>(kI) + ((size_t)b * N + jrow[g]) * RB;
            const uint8_t *kc = krow + kg * (DI / 8);
            if constexpr (RB % 8 == 0 && DI % 64 == 0 && (DI / 8) % 8 == 0) {
#pragma unroll
                for (int s = 0; s < KS; s += 2) {
                    const uint2 v = valid[g] ? *reinterpret_cast<const uint2 *>(kc + 4 * s) : make_uint2(0u, 0u);
                    kw4[g][s] = v.x;
                    kw4[g][s + 1] = v.y;
                }
            } else {
#pragma unroll
                for (int s = 0; s < KS; s++) kw4[g][s] = valid[g] ? *reinterpret_cast<const uint32_t *>(kc + 4 * s) : 0u;
            }
            const uint8_t *ksc = krow + DI / 2 + kg * (DI / 64);
            uint32_t sw = 0;
            if constexpr (DI / 64 == 4) sw = valid[g] ? *reinterpret_cast<const uint32_t *>(ksc) : 0u;
            else if constexpr (DI / 64 == 2) sw = valid[g] ? (uint32_t)*reinterpret_cast<const uint16_t *>(ksc) : 0u;
            else sw = valid[g] ? (uint32_t)*ksc : 0u;
#pragma unroll
            for (int s = 0; s < KS; s++) ks4[g][s] = (sw >> (8 * (s / 2))) & 0xffu;
        } else {
            const uint16_t *krow = kI + ((size_t)b * N + jrow[g]) * DI + 8 * kg;
#pragma unroll
            for (int s = 0; s < KS; s++)
                kb[g][s] = valid[g] ? *reinterpret_cast<const u32x4 *>(krow + 32 * s) : zero;
        }
    }
    // Query heads (A operand) and the weights of the result rows this lane holds.
    u32x4 qa[HT][KS];
    const uint16_t *qrow = qI + (size_t)bq * HI * DI;
#pragma unroll
    for (int ht = 0; ht < HT; ht++)
#pragma unroll
        for (int s = 0; s < KS; s++)
            qa[ht][s] = *reinterpret_cast<const u32x4 *>(qrow + (ht * 16 + col) * DI +
                                                        (KFP4 ? kg * (DI / 4) + 8 * s : 32 * s + 8 * kg));
    float wv[HT][4];
#pragma unroll
    for (int ht = 0; ht < HT; ht++)
#pragma unroll
        for (int r = 0; r < 4; r++) wv[ht][r] = w[(size_t)bq * HI + ht * 16 + 4 * kg + r];
    // sum_h |w_h| ||q_h|| in binary64 from the query fragments in registers,
    // while the key rows are in flight: in the query's first tile, wave x takes
    // head tiles x, x + 4, ..., and thread 0 adds the tiles' terms after the
    // tile statistics' barrier (a block-wide pass over the query rows at the
    // end of that tile held the launch open).  Fixed order: lane partials,
    // then kg pairs, then a butterfly over col, then ht.
    __shared__ double swq_sh[HT];
    if (sumwq && tile == 0) {
        const int wu = __builtin_amdgcn_readfirstlane(wave);
#pragma unroll
        for (int ht = 0; ht < HT; ht++) {
            if (ht % 4 != wu) continue;
            double q2 = 0.0;
#pragma unroll
            for (int s2 = 0; s2 < KS; s2++)
#pragma unroll
                for (int e = 0; e < 4; e++) {
                    const double x0 = (double)bf16_to_f32((uint16_t)(qa[ht][s2][e] & 0xffffu));
                    const double x1 = (double)bf16_to_f32((uint16_t)(qa[ht][s2][e] >> 16));
                    q2 = fma(x0, x0, q2);
                    q2 = fma(x1, x1, q2);
                }
            q2 += __shfl_xor(q2, 16);
            q2 += __shfl_xor(q2, 32);
            double t = fabs((double)w[(size_t)bq * HI + ht * 16 + col]) * sqrt(q2);
            for (int o = 1; o < 16; o <<= 1) t += __shfl_xor(t, o);
            if (lane == 0) swq_sh[ht] = t;
        }
    }

    float smin = POS_INF, smax = NEG_INF, kmax2 = 0.f;
    uint32_t nval = 0;
#pragma unroll
    for (int g = 0; g < G; g++) {
        if constexpr (KFP4) {
#pragma unroll
            for (int s = 0; s < KS; s++) kb[g][s] = fp4_keys_to_bf16x8<DI>(kw4[g][s], ks4[g][s]);
        }
        f32x4 acc[HT];
#pragma unroll
        for (int ht = 0; ht < HT; ht++) acc[ht] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int s = 0; s < KS; s++)
#pragma unroll
            for (int ht = 0; ht < HT; ht++)
                acc[ht] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, qa[ht][s]),
                                                                  __builtin_bit_cast(bf16x8, kb[g][s]), acc[ht], 0, 0,
                                                                  0);
        float part = 0.f;
#pragma unroll
        for (int ht = 0; ht < HT; ht++)
#pragma unroll
            for (int r = 0; r < 4; r++) part = fmaf(wv[ht][r], relu_bits(acc[ht][r]), part);
        part = bfly32(bfly16(part, OpAdd{}), OpAdd{});
        // squared norm of key row (l%16), from the B fragments already in registers
        float ss = 0.f;
#pragma unroll
        for (int s = 0; s < KS; s++)
#pragma unroll
            for (int e = 0; e < 4; e++) {
                bf16x2 v = __builtin_bit_cast(bf16x2, kb[g][s][e]);
                ss = __builtin_amdgcn_fdot2_f32_bf16(v, v, ss, false);
            }
        ss = bfly32(bfly16(ss, OpAdd{}), OpAdd{});
        const int64_t slot = slot0 + g * 16 + col;
        if (kg == 0 && slot < n) scores[(int64_t)bq * n + slot] = valid[g] ? part : NEG_INF;
        if (valid[g]) {
            smin = fminf(smin, part);
            smax = fmaxf(smax, part);
            kmax2 = fmaxf(kmax2, ss);
            nval += (kg == 0);
        }
    }
    reduce_tile_stat(smin, smax, nval, kmax2, stats + (size_t)bq * ntiles + tile);  // ends with a barrier
    if (sumwq && tile == 0 && threadIdx.x == 0) {
        double acc = 0.0;
#pragma unroll
        for (int ht = 0; ht < HT; ht++) acc += swq_sh[ht];
        sumwq[bq] = acc;
    }
}

// ----------------------------------------------------------- streaming path
// Same contraction and operand layouts as k_index_mfma, for full scans with
// many tiles.  A block's 4 waves take one 256-slot tile per pass, wave w its
// 64-slot step w, and the blocks of a query sweep the tiles together: in pass
// i block x takes tile x + nbx i (nbx = blocks per query), so at any moment
// the waves of a query read one compact region of the key cache (adjacent
// 64 KiB tiles) rather than 2048 scattered streams.  The key fragments of a
// 16-slot group are reloaded with the next pass's rows as soon as the
// group's matrix-core products are issued, so a wave keeps about 16 KiB of
// keys in flight with a single register buffer.  The query heads are read
// from HBM once per block (16 B per thread, issued ahead of the first key
// rows) and handed to the waves' fragments through LDS: loading them per
// wave straight from memory moved four times the bytes through the CU's
// load path before the first key rows went out.  The block's 1024 scores
// are kept in LDS and written after the last pass, in coalesced stores;
// each tile's statistics are the min / max / count of its 4 waves'
// reductions.
template <int HI, int DI, bool KFP4>
__global__ __launch_bounds__(256, 2) void k_index_stream(const uint16_t *__restrict__ qI, const float *__restrict__ w,
                                                         const uint16_t *__restrict__ kI, int Q, int64_t N,
                                                         const int64_t *__restrict__ q_pos, int m,
                                                         float *__restrict__ scores, TileStat *__restrict__ stats,
                                                         int ntiles, double *__restrict__ sumwq) {
    constexpr int HT = HI / 16;
    constexpr int KS = DI / 32;
    constexpr int G = 4;             // 16-slot groups per step
    constexpr int IT = 4;            // passes (tiles per block)
    static_assert(TILE == 4 * 64, "a tile is one 64-slot step per wave");
    constexpr int QN = HI * DI / 8, QPT = (QN + 255) / 256;  // 16-byte pieces of q, per thread
    __shared__ TileStat tst[IT][4];
    __shared__ float ssh[IT][TILE];
    __shared__ __attribute__((aligned(16))) uint16_t qsh[HI * DI];
    const int bq = blockIdx.y;
    const int b = bq / Q;
    const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
    const int col = lane & 15, kg = lane >> 4;
    const int64_t nvis = visible_entries(q_pos, bq, m, N);  // slots >= nvis are not scored
    const int nbx = gridDim.x;
    const int span = nbx * IT;
    // each query starts its sweep at its own offset, so that the queries'
    // regions (which sit a power of two apart) do not load the same memory
    // channels at the same time
    const int rot = (int)(((int64_t)bq * 8) % span);
    auto tile_of = [&](int it) {
        const int t = blockIdx.x + nbx * it + rot;
        return t < span ? t : t - span;
    };
    // this wave's first slot in pass it (tiles past the end read clamped rows and are dropped)
    auto step0 = [&](int it) { return (int64_t)tile_of(it) * TILE + wave * 64; };

    // Rows past the visible range are clamped to the last row of the key
    // cache and loaded anyway (no branch around the loads); their scores are
    // replaced by -inf and they take no part in the statistics.
    const uint16_t *kb0 = kI + (size_t)b * N * DI + 8 * kg;
    const int64_t last = N - 1;
    auto krow = [&](int it, int g) {
        const int64_t j = step0(it) + g * 16 + col;
        return kb0 + (size_t)(j < last ? j : last) * DI;
    };
    // FP4 keys: lane group kg holds channels kg DI/4 .. + DI/4 - 1 of its row
    // (contiguous code and scale bytes, see k_index_mfma), decoded to bf16 just
    // before the group's matrix-core steps
    constexpr int RB = DI / 2 + DI / 16;
    const uint8_t *kq0 = reinterpret_cast<const uint8_t *>(kI) + (size_t)b * N * RB;
    uint32_t kw[KFP4 ? G : 1][KS], kscl[KFP4 ? G : 1];
    auto load_fp4 = [&](int it, int g) {
        const int64_t j0 = step0(it) + g * 16 + col;
        const uint8_t *row = kq0 + (size_t)(j0 < last ? j0 : last) * RB;
        const uint8_t *kc = row + kg * (DI / 8);
        if constexpr (RB % 8 == 0 && (DI / 8) % 8 == 0) {
#pragma unroll
            for (int s = 0; s < KS; s += 2) {
                const uint2 v = *reinterpret_cast<const uint2 *>(kc + 4 * s);
                kw[g][s] = v.x;
                kw[g][s + 1] = v.y;
            }
        } else {
#pragma unroll
            for (int s = 0; s < KS; s++) kw[g][s] = *reinterpret_cast<const uint32_t *>(kc + 4 * s);
        }
        const uint8_t *ksc = row + DI / 2 + kg * (DI / 64);
        if constexpr (DI / 64 == 4) kscl[g] = *reinterpret_cast<const uint32_t *>(ksc);
        else if constexpr (DI / 64 == 2) kscl[g] = (uint32_t)*reinterpret_cast<const uint16_t *>(ksc);
        else kscl[g] = (uint32_t)*ksc;
    };
    // the query heads first, so that waiting for them never waits for key rows
    // (the guard is compiled out when the pieces split evenly over the block:
    // a conditional load would be sunk below the key loads)
    u32x4 qst[QPT];
    {
        const u32x4 *src = reinterpret_cast<const u32x4 *>(qI + (size_t)bq * HI * DI);
#pragma unroll
        for (int i = 0; i < QPT; i++)
            qst[i] = src[QN % 256 == 0 ? (int)threadIdx.x + 256 * i : min((int)threadIdx.x + 256 * i, QN - 1)];
    }
    __builtin_amdgcn_sched_barrier(0);
    f32x4 wv[HT];
#pragma unroll
    for (int ht = 0; ht < HT; ht++) wv[ht] = *reinterpret_cast<const f32x4 *>(w + (size_t)bq * HI + ht * 16 + 4 * kg);
    u32x4 kb[KFP4 ? 1 : G][KS];
#pragma unroll
    for (int g = 0; g < G; g++) {
        if constexpr (KFP4) {
            load_fp4(0, g);
        } else {
            const uint16_t *kr = krow(0, g);
#pragma unroll
            for (int s = 0; s < KS; s++) kb[g][s] = *reinterpret_cast<const u32x4 *>(kr + 32 * s);
        }
    }
#pragma unroll
    for (int i = 0; i < QPT; i++)
        if (QN % 256 == 0 || (int)threadIdx.x + 256 * i < QN) reinterpret_cast<u32x4 *>(qsh)[threadIdx.x + 256 * i] = qst[i];
    __syncthreads();
    u32x4 qa[HT][KS];
#pragma unroll
    for (int ht = 0; ht < HT; ht++)
#pragma unroll
        for (int s = 0; s < KS; s++)
            qa[ht][s] = *reinterpret_cast<const u32x4 *>(qsh + (ht * 16 + col) * DI +
                                                        (KFP4 ? kg * (DI / 4) + 8 * s : 32 * s + 8 * kg));
    if (sumwq && blockIdx.x == 0 && wave == 0) {
        // sum_h |w_h| ||q_h|| in binary64 from the query fragments in
        // registers (lane (col, kg) holds 8 KS elements of head 16 ht + col),
        // while the first key rows are in flight.  Fixed order: lane
        // partials, then kg pairs, then a butterfly over col, then ht.
        double acc = 0.0;
#pragma unroll
        for (int ht = 0; ht < HT; ht++) {
            double q2 = 0.0;
#pragma unroll
            for (int s2 = 0; s2 < KS; s2++)
#pragma unroll
                for (int e = 0; e < 4; e++) {
                    const double x0 = (double)bf16_to_f32((uint16_t)(qa[ht][s2][e] & 0xffffu));
                    const double x1 = (double)bf16_to_f32((uint16_t)(qa[ht][s2][e] >> 16));
                    q2 = fma(x0, x0, q2);
                    q2 = fma(x1, x1, q2);
                }
            q2 += __shfl_xor(q2, 16);
            q2 += __shfl_xor(q2, 32);
            double t = fabs((double)w[(size_t)bq * HI + ht * 16 + col]) * sqrt(q2);
            for (int o = 1; o < 16; o <<= 1) t += __shfl_xor(t, o);
            acc += t;
        }
        if (lane == 0) sumwq[bq] = acc;
    }

#pragma unroll
    for (int it = 0; it < IT; it++) {
        float part[G], ss[G];
#pragma unroll
        for (int g = 0; g < G; g++) {
            u32x4 kd[KS];  // this group's key fragments
#pragma unroll
            for (int s = 0; s < KS; s++) {
                if constexpr (KFP4) kd[s] = fp4_keys_to_bf16x8<DI>(kw[g][s], (kscl[g] >> (8 * (s / 2))) & 0xffu);
                else kd[s] = kb[g][s];
            }
            f32x4 acc[HT];
#pragma unroll
            for (int ht = 0; ht < HT; ht++) acc[ht] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
            for (int s = 0; s < KS; s++)
#pragma unroll
                for (int ht = 0; ht < HT; ht++)
                    acc[ht] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, qa[ht][s]),
                                                                      __builtin_bit_cast(bf16x8, kd[s]),
                                                                      acc[ht], 0, 0, 0);
            float q2 = 0.f;
#pragma unroll
            for (int s = 0; s < KS; s++)
#pragma unroll
                for (int e = 0; e < 4; e++) {
                    bf16x2 v = __builtin_bit_cast(bf16x2, kd[s][e]);
                    q2 = __builtin_amdgcn_fdot2_f32_bf16(v, v, q2, false);
                }
            ss[g] = q2;
            if (it + 1 < IT) {  // this group's rows of the next pass
                if constexpr (KFP4) {
                    load_fp4(it + 1, g);
                } else {
                    const uint16_t *kr = krow(it + 1, g);
#pragma unroll
                    for (int s = 0; s < KS; s++) kb[g][s] = *reinterpret_cast<const u32x4 *>(kr + 32 * s);
                }
            }
            float p = 0.f;
#pragma unroll
            for (int ht = 0; ht < HT; ht++)
#pragma unroll
                for (int r = 0; r < 4; r++) p = fmaf(wv[ht][r], relu_bits(acc[ht][r]), p);
            part[g] = p;
            // keep each group's reload where it is: hoisting them all would need a second buffer
            __builtin_amdgcn_sched_barrier(0);
        }
#pragma unroll
        for (int g = 0; g < G; g++) {
            part[g] = bfly32(bfly16(part[g], OpAdd{}), OpAdd{});
            ss[g] = bfly32(bfly16(ss[g], OpAdd{}), OpAdd{});
        }
        // lane l = 16 kg + col holds slot 64 w + l of the tile, i.e. group kg's row col
        const float mine = kg == 0 ? part[0] : kg == 1 ? part[1] : kg == 2 ? part[2] : part[3];
        const float mss = kg == 0 ? ss[0] : kg == 1 ? ss[1] : kg == 2 ? ss[2] : ss[3];
        const int64_t slot = step0(it) + lane;
        const bool ok = slot < nvis;
        ssh[it][wave * 64 + lane] = ok ? mine : NEG_INF;
        TileStat t;
        t.smin = wave_min(ok ? mine : POS_INF);
        t.smax = wave_max(ok ? mine : NEG_INF);
        t.kmax2 = wave_max(ok ? mss : 0.f);
        t.nvalid = (uint32_t)__builtin_popcountll(__ballot(ok));
        if (lane == 0) tst[it][wave] = t;
    }
    __syncthreads();
#pragma unroll
    for (int it = 0; it < IT; it++) {
        const int64_t slot = (int64_t)tile_of(it) * TILE + threadIdx.x;
        if (slot < N) scores[(int64_t)bq * N + slot] = ssh[it][threadIdx.x];
    }
    if (threadIdx.x < IT) {
        const int it = threadIdx.x;
        const int tile = tile_of(it);
        if (tile < ntiles) {
            TileStat t = tst[it][0];
#pragma unroll
            for (int x = 1; x < 4; x++) {
                const TileStat u = tst[it][x];
                t.smin = fminf(t.smin, u.smin);
                t.smax = fmaxf(t.smax, u.smax);
                t.kmax2 = fmaxf(t.kmax2, u.kmax2);
                t.nvalid += u.nvalid;
            }
            stats[(size_t)bq * ntiles + tile] = t;
        }
    }
}

// ---------------------------------------------------------------- VALU path
// Any head count / dim / dtype: one slot per thread, fp32 FMA in sequential
// order, query heads staged in LDS as fp32.
// One slot's score: fp32 FMAs in sequential order (d, then h), the key
// element type fixed per instantiation so that the unrolled loop has its key
// loads in flight together rather than one dependent load per step.
template <bool F32>
__device__ __forceinline__ void valu_slot_score(const float *qs, const float *wq, const void *kI, size_t base, int HI,
                                                int dI, float &s, float &ss) {
    for (int h = 0; h < HI; h++) {
        float dot = 0.f;
#pragma unroll 8
        for (int d = 0; d < dI; d++) {
            const float kv = F32 ? static_cast<const float *>(kI)[base + d]
                                 : bf16_to_f32(static_cast<const uint16_t *>(kI)[base + d]);
            dot = fmaf(qs[h * dI + d], kv, dot);
            if (h == 0) ss = fmaf(kv, kv, ss);
        }
        s = fmaf(wq[h], fmaxf(dot, 0.f), s);
    }
}

__global__ __launch_bounds__(256) void k_index_valu(const void *__restrict__ qI, int dt, const float *__restrict__ w,
                                                    const void *__restrict__ kI, int Q, int HI, int dI, int64_t N,
                                                    const int64_t *__restrict__ q_pos, int m,
                                                    const int32_t *__restrict__ cand, int P,
                                                    float *__restrict__ scores, TileStat *__restrict__ stats,
                                                    int ntiles, double *__restrict__ sumwq) {
    extern __shared__ float qs[];  // [HI * dI]
    const int bq = blockIdx.y;
    const int b = bq / Q;
    const int64_t n = cand ? (int64_t)P : N;
    const int64_t nvis = visible_entries(q_pos, bq, m, N);
    const int HD = HI * dI;
    for (int i = threadIdx.x; i < HD; i += blockDim.x) {
        size_t off = (size_t)bq * HD + i;
        qs[i] = dt == CSA2_F32 ? static_cast<const float *>(qI)[off] : bf16_to_f32(static_cast<const uint16_t *>(qI)[off]);
    }
    __syncthreads();
    const int64_t slot = (int64_t)blockIdx.x * TILE + threadIdx.x;
    int64_t j = -1;
    if (slot < n) j = cand ? (int64_t)cand[(int64_t)bq * P + slot] : slot;
    const bool valid = (j >= 0) && (j < nvis);
    float s = 0.f, ss = 0.f;
    if (valid) {
        const size_t base = ((size_t)b * N + j) * dI;
        if (dt == CSA2_F32) valu_slot_score<true>(qs, w + (size_t)bq * HI, kI, base, HI, dI, s, ss);
        else valu_slot_score<false>(qs, w + (size_t)bq * HI, kI, base, HI, dI, s, ss);
    }
    if (slot < n) scores[(int64_t)bq * n + slot] = valid ? s : NEG_INF;
    reduce_tile_stat(valid ? s : POS_INF, valid ? s : NEG_INF, valid ? 1u : 0u, valid ? ss : 0.f,
                     stats + (size_t)bq * ntiles + blockIdx.x);
    if (sumwq && blockIdx.x == 0) {
        __shared__ double dred[256 / 16];
        const double v = block_sumwq<256>(qI, dt, w, HI, dI, bq, dred);
        if (threadIdx.x == 0) sumwq[bq] = v;
    }
}

// ------------------------------------------------------------- error bound
// E = 2^-22 (dI + HI + 2) * max_j ||k_j|| * sum_h |w_h| ||q_h||  (+ tiny).
// Derivation: each fp32 product of bf16/fp32 inputs is exact; each fp32
// accumulation in the dot product (<= dI steps, any order, rounding or
// truncating) and in the weighted head sum (<= HI + 2 steps) is charged a
// relative error of 2^-23; the total is bounded through Cauchy-Schwarz by
// (dI + HI + 1) 2^-23 sum_h |w_h| ||q_h|| ||k_j||, and the binary64 reference
// differs from the exact value by far less.  2^-22 doubles the whole budget.
// max ||k||^2 comes from fp32 sums (relative error < dI 2^-23) and is widened
// by 2^-10 before the square root.
__global__ __launch_bounds__(256) void k_err_bound(const void *__restrict__ qI, int dt, const float *__restrict__ w,
                                                   int HI, int dI, const TileStat *__restrict__ stats, int ntiles,
                                                   float *__restrict__ err32, double *__restrict__ err64) {
    __shared__ double dred[256 / 16];
    __shared__ float kred[4];
    const int bq = blockIdx.x;
    float km = 0.f;
    for (int t = threadIdx.x; t < ntiles; t += 256) km = fmaxf(km, stats[(size_t)bq * ntiles + t].kmax2);
    km = wave_max(km);
    if ((threadIdx.x & 63) == 0) kred[threadIdx.x >> 6] = km;
    const double sumwq = block_sumwq<256>(qI, dt, w, HI, dI, bq, dred);  // has barriers
    if (threadIdx.x == 0) {
        const float k2 = fmaxf(fmaxf(kred[0], kred[1]), fmaxf(kred[2], kred[3]));
        const double E = score_bound(sqrt((double)k2 * (1.0 + ldexp(1.0, -10))), sumwq * (1.0 + ldexp(1.0, -30)), HI, dI);
        if (err64) err64[bq] = E;
        if (err32) {
            float e = (float)E;
            if ((double)e < E) e = nextafterf(e, POS_INF);
            err32[bq] = e;
        }
    }
}

// Registers of the streaming kernel: query fragments HI*DI/128 plus key
// fragments DI/2.
constexpr bool stream_fits(int HI, int DI) { return HI * DI / 128 + DI / 2 <= 128; }
constexpr int64_t STREAM_MIN_TILES = 1024;  // below this, one tile per block fills the chip better

// ------------------------------------------------------------ prefill path
// A prefill chunk scores thousands of query tokens against the same keys, so
// the score is one dense contraction [queries x heads] x [keys] and the keys
// are what to reuse.  Block = one 256-key tile x PF_QT query tokens of one
// sequence: each wave loads the bf16 B fragments of its 64 keys once (and
// their squared norms), then takes the block's queries in turn, each
// query's heads (A fragments) read from LDS, where the next query is staged
// (global -> registers -> the other LDS buffer) while this one is scored.  The
// contraction, the ReLU-weighted head sum and its order are those of
// k_index_mfma, so the scores are the same bits.  Per query and tile the
// waves' statistics meet in LDS and are written at the end; tile 0's blocks
// also write each query's sum_h |w_h| ||q_h||.
constexpr int PF_QT = 32;      // query tokens per block
constexpr int PF_MIN_Q = 64;   // query tokens per sequence from which the chunk path is taken

template <int HI, int DI>
__global__ __launch_bounds__(256, 2) void k_index_prefill(const uint16_t *__restrict__ qI, const float *__restrict__ w,
                                                          const uint16_t *__restrict__ kI, int Q, int64_t N,
                                                          const int64_t *__restrict__ q_pos, int m,
                                                          float *__restrict__ scores, TileStat *__restrict__ stats,
                                                          int ntiles, double *__restrict__ sumwq) {
    constexpr int HT = HI / 16, KS = DI / 32, G = 4;
    constexpr int QE = HI * DI;                 // bf16 elements of one query token's heads
    constexpr int QPT = QE / 8 / 256;           // 16-byte pieces per thread
    static_assert(QE % (8 * 256) == 0, "a query's heads split evenly over the block");
    constexpr int QRS = DI + 8;                 // LDS row stride of a head (16-byte pad: no bank conflicts)
    __shared__ __attribute__((aligned(16))) uint16_t qs[2][HI * QRS];
    __shared__ float wsh[2][HI];
    __shared__ f32x4 stp[PF_QT][4];             // per query and wave: smin, smax, kmax2, count
    __shared__ int64_t nvis_sh[PF_QT];          // per query: visible slots (one 64-bit division each, once)
    const int tile = blockIdx.x;
    const int qtiles = (Q + PF_QT - 1) / PF_QT;
    const int b = blockIdx.y / qtiles;
    const int q0 = (blockIdx.y % qtiles) * PF_QT;
    const int nq = min(PF_QT, Q - q0);
    const int bq0 = b * Q + q0;
    const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
    const int col = lane & 15, kg = lane >> 4;
    const int64_t slot0 = (int64_t)tile * TILE + wave * 64;

    // this wave's keys: B fragments and squared norms (rows past N read as 0)
    u32x4 kb[G][KS];
    float kn[G];
    {
        const u32x4 zero = {0u, 0u, 0u, 0u};
#pragma unroll
        for (int g = 0; g < G; g++) {
            const int64_t j = slot0 + g * 16 + col;
            const uint16_t *kr = kI + ((size_t)b * N + (j < N ? j : 0)) * DI + 8 * kg;
#pragma unroll
            for (int s2 = 0; s2 < KS; s2++) kb[g][s2] = j < N ? *reinterpret_cast<const u32x4 *>(kr + 32 * s2) : zero;
        }
    }
    // query 0 of the block into buffer 0
    auto load_q = [&](int qi, u32x4 (&reg)[QPT], float &wreg) {
        const u32x4 *src = reinterpret_cast<const u32x4 *>(qI + (size_t)(bq0 + qi) * QE);
#pragma unroll
        for (int i = 0; i < QPT; i++) reg[i] = src[threadIdx.x + 256 * i];
        wreg = threadIdx.x < HI ? w[(size_t)(bq0 + qi) * HI + threadIdx.x] : 0.f;
    };
    auto put_q = [&](int buf, const u32x4 (&reg)[QPT], float wreg) {
#pragma unroll
        for (int i = 0; i < QPT; i++) {
            const int pc = threadIdx.x + 256 * i;  // 16-byte piece: head pc / (DI / 8), channels 8 (pc % (DI / 8)) ..
            *reinterpret_cast<u32x4 *>(qs[buf] + (pc / (DI / 8)) * QRS + 8 * (pc % (DI / 8))) = reg[i];
        }
        if (threadIdx.x < HI) wsh[buf][threadIdx.x] = wreg;
    };
    // queries in flight two ahead: query qi + 1 waits in registers (set
    // (qi + 1) & 1) while qi is scored, and qi + 2 is requested into the set
    // qi just left; both sets are named statically (the loop is unrolled by 2)
    u32x4 qr[2][QPT];
    float wr[2] = {0.f, 0.f};
    load_q(0, qr[0], wr[0]);
    if (nq > 1) load_q(1, qr[1], wr[1]);
#pragma unroll
    for (int g = 0; g < G; g++) {
        float ss = 0.f;
#pragma unroll
        for (int s2 = 0; s2 < KS; s2++)
#pragma unroll
            for (int e = 0; e < 4; e++) {
                bf16x2 v = __builtin_bit_cast(bf16x2, kb[g][s2][e]);
                ss = __builtin_amdgcn_fdot2_f32_bf16(v, v, ss, false);
            }
        kn[g] = bfly32(bfly16(ss, OpAdd{}), OpAdd{});
    }
    put_q(0, qr[0], wr[0]);
    if ((int)threadIdx.x < nq) nvis_sh[threadIdx.x] = visible_entries(q_pos, bq0 + threadIdx.x, m, N);

    auto score_query = [&](int qi) {
        const int buf = qi & 1;
        const int bq = bq0 + qi;
        const int64_t nvis = nvis_sh[qi];
        u32x4 qa[HT][KS];
#pragma unroll
        for (int ht = 0; ht < HT; ht++)
#pragma unroll
            for (int s2 = 0; s2 < KS; s2++)
                qa[ht][s2] = *reinterpret_cast<const u32x4 *>(qs[buf] + (ht * 16 + col) * QRS + 32 * s2 + 8 * kg);
        float wv[HT][4];
#pragma unroll
        for (int ht = 0; ht < HT; ht++)
#pragma unroll
            for (int r = 0; r < 4; r++) wv[ht][r] = wsh[buf][ht * 16 + 4 * kg + r];
        float smin = POS_INF, smax = NEG_INF, kmax2 = 0.f, cnt = 0.f;
        // this lane's slots are slot0 + col + 16 g: visible below rem_vis, stored below rem_n
        const int64_t own = slot0 + col;
        const int rem_vis = (int)max<int64_t>(min<int64_t>(nvis - own, 1 << 20), -1);
        const int rem_n = (int)max<int64_t>(min<int64_t>(N - own, 1 << 20), -1);
        float *srow = scores + (size_t)bq * N + own;
#pragma unroll
        for (int g = 0; g < G; g++) {
            f32x4 acc[HT];
#pragma unroll
            for (int ht = 0; ht < HT; ht++) acc[ht] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
            for (int s2 = 0; s2 < KS; s2++)
#pragma unroll
                for (int ht = 0; ht < HT; ht++)
                    acc[ht] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, qa[ht][s2]),
                                                                      __builtin_bit_cast(bf16x8, kb[g][s2]), acc[ht], 0,
                                                                      0, 0);
            float part = 0.f;
#pragma unroll
            for (int ht = 0; ht < HT; ht++)
#pragma unroll
                for (int r = 0; r < 4; r++) part = fmaf(wv[ht][r], relu_bits(acc[ht][r]), part);
            part = bfly32(bfly16(part, OpAdd{}), OpAdd{});
            const bool valid = g * 16 < rem_vis;
            if (kg == 0 && g * 16 < rem_n) srow[g * 16] = valid ? part : NEG_INF;
            if (valid) {
                smin = fminf(smin, part);
                smax = fmaxf(smax, part);
                kmax2 = fmaxf(kmax2, kn[g]);
                cnt += 1.f;
            }
        }
        // the wave's statistics: every kg group holds the same values
        smin = bfly8(bfly4(bfly2(bfly1(smin, OpMin{}), OpMin{}), OpMin{}), OpMin{});
        smax = bfly8(bfly4(bfly2(bfly1(smax, OpMax{}), OpMax{}), OpMax{}), OpMax{});
        kmax2 = bfly8(bfly4(bfly2(bfly1(kmax2, OpMax{}), OpMax{}), OpMax{}), OpMax{});
        cnt = bfly8(bfly4(bfly2(bfly1(cnt, OpAdd{}), OpAdd{}), OpAdd{}), OpAdd{});
        if (lane == 0) stp[qi][wave] = f32x4{smin, smax, kmax2, cnt};
    };
    for (int q2 = 0; q2 < nq; q2 += 2) {
#pragma unroll
        for (int h = 0; h < 2; h++) {
            const int qi = q2 + h;
            if (qi < nq) {
                __syncthreads();  // query qi staged in buffer qi & 1; the other buffer free
                if (qi + 2 < nq) load_q(qi + 2, qr[h], wr[h]);
                score_query(qi);
                if (qi + 1 < nq) put_q(h ^ 1, qr[h ^ 1], wr[h ^ 1]);
            }
        }
    }
    __syncthreads();
    if ((int)threadIdx.x < nq) {
        const int qi = threadIdx.x;
        TileStat t;
        t.smin = fminf(fminf(stp[qi][0][0], stp[qi][1][0]), fminf(stp[qi][2][0], stp[qi][3][0]));
        t.smax = fmaxf(fmaxf(stp[qi][0][1], stp[qi][1][1]), fmaxf(stp[qi][2][1], stp[qi][3][1]));
        t.kmax2 = fmaxf(fmaxf(stp[qi][0][2], stp[qi][1][2]), fmaxf(stp[qi][2][2], stp[qi][3][2]));
        t.nvalid = (uint32_t)(stp[qi][0][3] + stp[qi][1][3] + stp[qi][2][3] + stp[qi][3][3]);
        stats[(size_t)(bq0 + qi) * ntiles + tile] = t;
    }
    // sum_h |w_h| ||q_h|| of the block's query tokens, one per key tile: the
    // block of tile x takes token x (and x + ntiles, ...).  All of them in the
    // first tile's block held that block, and with it the launch, back by a
    // serial loop over 32 tokens.
    if (sumwq) {
        __shared__ double dred[256 / 16];
        for (int qi = tile; qi < nq; qi += (int)gridDim.x) {
            const double v = block_sumwq<256>(qI, CSA2_BF16, w, HI, DI, bq0 + qi, dred);
            if (threadIdx.x == 0) sumwq[bq0 + qi] = v;
        }
    }
}

template <int HI, int DI>
void launch_mfma(const void *qI, const float *w, const void *kI, int B, int Q, int64_t N, const int64_t *q_pos,
                 int m, const int32_t *cand, int P, float *scores, TileStat *stats, int ntiles, double *sumwq,
                 bool kfp4, hipStream_t s) {
    if (kfp4) {
        if constexpr (DI % 64 == 0) {
            if constexpr (stream_fits(HI, DI)) {
                if (!cand && (int64_t)B * Q * ntiles >= STREAM_MIN_TILES) {
                    dim3 grid((ntiles + 3) / 4, B * Q);
                    hipLaunchKernelGGL((k_index_stream<HI, DI, true>), grid, dim3(256), 0, s,
                                       static_cast<const uint16_t *>(qI), w, static_cast<const uint16_t *>(kI), Q, N,
                                       q_pos, m, scores, stats, ntiles, sumwq);
                    return;
                }
            }
            dim3 grid(ntiles, B * Q);
            hipLaunchKernelGGL((k_index_mfma<HI, DI, true>), grid, dim3(256), 0, s, static_cast<const uint16_t *>(qI),
                               w, static_cast<const uint16_t *>(kI), Q, N, q_pos, m, cand, P, scores, stats, ntiles,
                               sumwq);
        }
        return;
    }
    if constexpr (HI == 64 && DI == 128) {
        if (!cand && Q >= PF_MIN_Q) {
            dim3 grid(ntiles, B * ((Q + PF_QT - 1) / PF_QT));
            hipLaunchKernelGGL((k_index_prefill<HI, DI>), grid, dim3(256), 0, s, static_cast<const uint16_t *>(qI), w,
                               static_cast<const uint16_t *>(kI), Q, N, q_pos, m, scores, stats, ntiles, sumwq);
            return;
        }
    }
    if constexpr (stream_fits(HI, DI)) {
        if (!cand && (int64_t)B * Q * ntiles >= STREAM_MIN_TILES) {
            dim3 grid((ntiles + 3) / 4, B * Q);
            hipLaunchKernelGGL((k_index_stream<HI, DI, false>), grid, dim3(256), 0, s, static_cast<const uint16_t *>(qI), w,
                               static_cast<const uint16_t *>(kI), Q, N, q_pos, m, scores, stats, ntiles, sumwq);
            return;
        }
    }
    dim3 grid(ntiles, B * Q);
    hipLaunchKernelGGL((k_index_mfma<HI, DI, false>), grid, dim3(256), 0, s, static_cast<const uint16_t *>(qI), w,
                       static_cast<const uint16_t *>(kI), Q, N, q_pos, m, cand, P, scores, stats, ntiles, sumwq);
}

// FP4 indexer queries ("读完这篇，你就搞懂 DeepSeek v4 了", the passage on V4's
// FP4 quantization-aware training: the indexer's q is FP4 as well as its K):
// each query row is decoded once, exactly, into bf16 (piece t = 8 channels:
// 4 code bytes and their scale byte to 16 bytes), so that the scoring and
// the certified selection run on the bf16-query, FP4-key path unchanged.
__global__ __launch_bounds__(256) void k_fp4_rows_to_bf16(const uint8_t *__restrict__ rows, int64_t npieces, int D,
                                                          uint16_t *__restrict__ out) {
    const int64_t t = (int64_t)blockIdx.x * 256 + threadIdx.x;
    if (t >= npieces) return;
    const int ppr = D / 8;
    const int64_t r = t / ppr;
    const int c = (int)(t - r * ppr);
    const uint8_t *row = rows + r * (D / 2 + D / 16);
    const uint32_t word = *reinterpret_cast<const uint32_t *>(row + 4 * c);
    *reinterpret_cast<u32x4 *>(out + r * D + 8 * c) = fp4_keys_to_bf16x8<64>(word, row[D / 2 + c / 2]);
}

}  // namespace

bool index_mfma_supported(int dt, int HI, int dI) {
    if (dt != CSA2_BF16 && !(dt == CSA2_FP4 && dI % 64 == 0)) return false;
    switch (HI * 1000 + dI) {
        case 16032: case 16064: case 16128: case 16256:
        case 32032: case 32064: case 32128: case 32256:
        case 64032: case 64064: case 64128:
        case 128064:
            return true;
        default:
            return false;
    }
}

bool index_valu_supported(int HI, int dI) { return (int64_t)HI * dI <= 16384; }

void launch_index_score(const void *qI, int dt, const float *w, const void *kI, int B, int Q, int HI, int dI,
                        int64_t N, const int64_t *q_pos, int m, const int32_t *cand, int P, float *scores,
                        TileStat *stats, double *sumwq, hipStream_t s) {
    const int64_t n = cand ? (int64_t)P : N;
    const int ntiles = (int)((n + TILE - 1) / TILE);
    if (index_mfma_supported(dt, HI, dI)) {
#define CSA2_IDX_CASE(h, d)                                                                        \
    case h * 1000 + d:                                                                              \
        launch_mfma<h, d>(qI, w, kI, B, Q, N, q_pos, m, cand, P, scores, stats, ntiles, sumwq, dt == CSA2_FP4, s); \
        break;
        switch (HI * 1000 + dI) {
            CSA2_IDX_CASE(16, 32) CSA2_IDX_CASE(16, 64) CSA2_IDX_CASE(16, 128) CSA2_IDX_CASE(16, 256)
            CSA2_IDX_CASE(32, 32) CSA2_IDX_CASE(32, 64) CSA2_IDX_CASE(32, 128) CSA2_IDX_CASE(32, 256)
            CSA2_IDX_CASE(64, 32) CSA2_IDX_CASE(64, 64) CSA2_IDX_CASE(64, 128)
            CSA2_IDX_CASE(128, 64)
        }
#undef CSA2_IDX_CASE
    } else {
        dim3 grid(ntiles, B * Q);
        size_t lds = sizeof(float) * (size_t)HI * dI;
        hipLaunchKernelGGL(k_index_valu, grid, dim3(256), lds, s, qI, dt, w, kI, Q, HI, dI, N, q_pos, m, cand, P,
                           scores, stats, ntiles, sumwq);
    }
    check_launch("index score");
}

void launch_fp4_rows_to_bf16(const void *rows, int64_t nrows, int D, uint16_t *out, hipStream_t s) {
    const int64_t np = nrows * (D / 8);
    hipLaunchKernelGGL(k_fp4_rows_to_bf16, dim3((unsigned)((np + 255) / 256)), dim3(256), 0, s,
                       static_cast<const uint8_t *>(rows), np, D, out);
    check_launch("FP4 query decode");
}

void launch_err_bound(const void *qI, int dt, const float *w, int BQ, int HI, int dI, const TileStat *stats,
                      int ntiles, float *err32, double *err64, hipStream_t s) {
    const int qdt = dt == CSA2_FP4 ? CSA2_BF16 : dt;  // FP4 keys come with bf16 queries
    hipLaunchKernelGGL(k_err_bound, dim3(BQ), dim3(256), 0, s, qI, qdt, w, HI, dI, stats, ntiles, err32, err64);
    check_launch("error bound");
}

}  // namespace csa2
