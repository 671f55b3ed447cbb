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
// Matrix-core kernel (k_attn_split): a block serves one query over a fixed
// split of 128 selected entries (the split depends only on k, so a query's
// result does not depend on the batch) for 16 to 64 of its heads.  All rows
// of the split are gathered at once and staged in LDS as bf16 (FP4 rows
// decoded on the way in, to fp16, where they are also exact); S^T = C Q^T and
// O^T = C^T P^T run on the 16x16x32 matrix-core instruction of that type with
// the block's queries held in registers, a softmax over the split in between.
// Splits are merged by a small combine kernel.
#include "internal.h"

namespace csa2 {

// Selected entries per split: fixed, so that a query's result does not depend
// on the batch it is computed in.
constexpr int ATT_SPLIT = 128;
// Query tokens per sequence from which a call counts as a prefill chunk.
constexpr int ATT_TILES_MIN_Q = 64;

namespace {

constexpr float NEG_INF = -__builtin_inff();

// 4-bit E2M1 code -> binary32 bits (OCP MX element: bias 1, code 0bS001 = 0.5).
__device__ __forceinline__ uint32_t e2m1_bits(uint32_t c) {
    const uint32_t e = (c >> 1) & 3u, mb = c & 1u;
    const uint32_t mag = e ? (((e + 126u) << 23) | (mb << 22)) : (mb ? 0x3f000000u : 0u);
    return mag | ((c & 8u) << 28);
}
// FP4 row scale byte -> float: its E4M3 ("FN") value, the NaN code
// S.1111.111 saturating to +-448 (branch-free, see e4m3_mag_bits).
__device__ __forceinline__ float e4m3_val(uint32_t s) {
    return __uint_as_float(e4m3_mag_bits(s) | ((s & 0x80u) << 24));
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


// ------------------------------------------------------ operand helpers
typedef short __attribute__((ext_vector_type(4))) s16x4;
typedef float __attribute__((ext_vector_type(2))) f32x2;
typedef __bf16 __attribute__((ext_vector_type(2))) bf16x2v;  // converted to with round-to-nearest-even
typedef _Float16 __attribute__((ext_vector_type(2))) f16x2;

// 8 FP4 channels (one code word) with their E4M3 scale -> 8 fp16 values.  The
// conversion instruction applies the scale's power of two, an fp16 multiply
// its mantissa (1 + m/8, at most 3 bits); every product has <= 5 significant
// bits and a magnitude in [2^-10, 2688], so both steps are exact.
__device__ __forceinline__ u32x4 fp4_word_to_f16x8(uint32_t word, uint32_t sbyte) {
    const uint32_t mag = e4m3_mag_bits(sbyte);
    const float pow2 = __uint_as_float(mag ? mag & 0x7f800000u : 0x3f800000u);
    const uint32_t fbits = mag ? 0x3c00u | ((mag >> 13) & 0x3ffu) | ((sbyte & 0x80u) << 8) : 0u;
    const f16x2 f = __builtin_bit_cast(f16x2, fbits | (fbits << 16));
    const f16x2 v0 = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(word, pow2, 0) * f;
    const f16x2 v1 = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(word, pow2, 1) * f;
    const f16x2 v2 = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(word, pow2, 2) * f;
    const f16x2 v3 = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(word, pow2, 3) * f;
    return u32x4{__builtin_bit_cast(uint32_t, v0), __builtin_bit_cast(uint32_t, v1), __builtin_bit_cast(uint32_t, v2),
                 __builtin_bit_cast(uint32_t, v3)};
}

// ----------------------------------------------------------- split merge
// One thread per 8 channels of one head.  Up to COMB_UNROLL splits are read in
// one round of loads (their maxima, sums, scales and 8-channel fp16 partial
// rows, 16 bytes each), so the merge waits for memory once; more splits take
// further rounds, the running maximum rescaling what is already summed.
constexpr int COMB_UNROLL = 16;
constexpr int COMB_CPT = 8;  // channels per thread (a quarter of D is a multiple of 8 for D >= 32)

__global__ __launch_bounds__(256) void k_attn_combine(const uint16_t *__restrict__ part_o,
                                                      const float2 *__restrict__ part_ml,
                                                      const float *__restrict__ part_sc, int BQ, int H, int D,
                                                      int nsplit, void *__restrict__ out, int out_dt,
                                                      float *__restrict__ lse) {
    const int tpr = D / COMB_CPT;  // threads per head row
    const int64_t gid = (int64_t)blockIdx.x * 256 + threadIdx.x;
    const int64_t row = gid / tpr;  // (bq, h)
    const int c8 = (int)(gid % tpr);
    if (row >= (int64_t)BQ * H) return;
    const int64_t bqr = row / H;
    const int hr = (int)(row % H);
    const int quarter = COMB_CPT * c8 / (D / 4);  // the channels' scale slot
    float M = NEG_INF, Ls = 0.f;
    f32x4 acc0 = {0.f, 0.f, 0.f, 0.f}, acc1 = {0.f, 0.f, 0.f, 0.f};
    for (int s0 = 0; s0 < nsplit; s0 += COMB_UNROLL) {
        float2 ml[COMB_UNROLL];
        float sc[COMB_UNROLL];
        uint4 ph[COMB_UNROLL];
#pragma unroll
        for (int u = 0; u < COMB_UNROLL; u++) {
            // splits past the end read the last one and are dropped
            const size_t pi = ((size_t)bqr * nsplit + (s0 + u < nsplit ? s0 + u : nsplit - 1)) * H + hr;
            ml[u] = part_ml[pi];
            sc[u] = part_sc[pi * 4 + quarter];
            ph[u] = reinterpret_cast<const uint4 *>(part_o + pi * D)[c8];
        }
        float Mn = M;
#pragma unroll
        for (int u = 0; u < COMB_UNROLL; u++)
            if (s0 + u < nsplit) Mn = fmaxf(Mn, ml[u].x);
        if (Mn != NEG_INF) {
            if (M != NEG_INF && M != Mn) {
                const float f = __expf(M - Mn);
                Ls *= f;
                acc0 = acc0 * f;
                acc1 = acc1 * f;
            }
#pragma unroll
            for (int u = 0; u < COMB_UNROLL; u++)
                if (s0 + u < nsplit && ml[u].x != NEG_INF) {
                    const float f = __expf(ml[u].x - Mn);
                    Ls += ml[u].y * f;
                    const f16x2 a = __builtin_bit_cast(f16x2, ph[u].x), b = __builtin_bit_cast(f16x2, ph[u].y);
                    const f16x2 c = __builtin_bit_cast(f16x2, ph[u].z), d = __builtin_bit_cast(f16x2, ph[u].w);
                    const f32x4 p0 = {(float)a[0], (float)a[1], (float)b[0], (float)b[1]};
                    const f32x4 p1 = {(float)c[0], (float)c[1], (float)d[0], (float)d[1]};
                    const float fs = f * sc[u];
                    acc0 = acc0 + p0 * fs;
                    acc1 = acc1 + p1 * fs;
                }
            M = Mn;
        }
    }
    const float inv = Ls > 0.f ? 1.f / Ls : 0.f;
    const size_t oi = (size_t)row * D + COMB_CPT * c8;
    if (out_dt == CSA2_F32) {
        f32x4 *o = reinterpret_cast<f32x4 *>(static_cast<float *>(out) + oi);
        o[0] = acc0 * inv;
        o[1] = acc1 * inv;
    } else {
        uint4 w;
        w.x = uint32_t(f32_to_bf16_rne(acc0[0] * inv)) | (uint32_t(f32_to_bf16_rne(acc0[1] * inv)) << 16);
        w.y = uint32_t(f32_to_bf16_rne(acc0[2] * inv)) | (uint32_t(f32_to_bf16_rne(acc0[3] * inv)) << 16);
        w.z = uint32_t(f32_to_bf16_rne(acc1[0] * inv)) | (uint32_t(f32_to_bf16_rne(acc1[1] * inv)) << 16);
        w.w = uint32_t(f32_to_bf16_rne(acc1[2] * inv)) | (uint32_t(f32_to_bf16_rne(acc1[3] * inv)) << 16);
        *reinterpret_cast<uint4 *>(static_cast<uint16_t *>(out) + oi) = w;
    }
    if (lse && c8 == 0) lse[row] = Ls > 0.f ? M + logf(Ls) : NEG_INF;
}

// ------------------------------------------------------------ VALU kernel
// Any head count, dim and format: one block per (query, head), fp32 math.
// The logits of entries t0, t0 + 256, ... and O = sum p C over a fixed KV
// element type (FMT), so that the unrolled loops keep their row loads in
// flight together; loads are unconditional (a skipped entry reads row 0) and
// only the arithmetic is masked.
template <int FMT>
__device__ __forceinline__ float valu_logits(const float *qs, const uint8_t *kvb, int64_t rb, int D, int64_t N,
                                             const int32_t *irow, int k, float scale, float *as) {
    float mx = NEG_INF;
    for (int t = threadIdx.x; t < k; t += 256) {
        const int32_t j = irow[t];
        const bool ok = j >= 0 && j < N;
        const uint8_t *row = kvb + (size_t)(ok ? j : 0) * rb;
        float dot = 0.f;
#pragma unroll 8
        for (int d = 0; d < D; d++) dot = fmaf(qs[d], kv_elem(row, FMT, D, d), dot);
        const float a = ok ? scale * dot : NEG_INF;
        as[t] = a;
        mx = fmaxf(mx, a);
    }
    return mx;
}
template <int FMT>
__device__ __forceinline__ float valu_out(const uint8_t *kvb, int64_t rb, int D, int64_t N, const int32_t *irow,
                                          int k, const float *as, int d) {
    float acc = 0.f;
#pragma unroll 8
    for (int t = 0; t < k; t++) {
        const int32_t j = irow[t];
        const bool ok = j >= 0 && j < N;
        const float v = kv_elem(kvb + (size_t)(ok ? j : 0) * rb, FMT, D, d);
        if (ok && as[t] != 0.f) acc = fmaf(as[t], v, acc);
    }
    return acc;
}

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
    float mx = kv_dt == CSA2_F32    ? valu_logits<CSA2_F32>(qs, kvb, rb, D, N, irow, k, scale, as)
               : kv_dt == CSA2_BF16 ? valu_logits<CSA2_BF16>(qs, kvb, rb, D, N, irow, k, scale, as)
                                    : valu_logits<CSA2_FP4>(qs, kvb, rb, D, N, irow, k, scale, as);
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
        const float acc = kv_dt == CSA2_F32    ? valu_out<CSA2_F32>(kvb, rb, D, N, irow, k, as, d)
                          : kv_dt == CSA2_BF16 ? valu_out<CSA2_BF16>(kvb, rb, D, N, irow, k, as, d)
                                               : valu_out<CSA2_FP4>(kvb, rb, D, N, irow, k, as, d);
        const float v = Z > 0.f ? acc / Z : 0.f;
        if (q_dt == CSA2_F32) static_cast<float *>(out)[qoff + d] = v;
        else static_cast<uint16_t *>(out)[qoff + d] = f32_to_bf16_rne(v);
    }
    if (lse && threadIdx.x == 0) lse[(size_t)bq * H + h] = Z > 0.f ? M + logf(Z) : NEG_INF;
}

// ------------------------------------------- selection finish (per block)
// The certified top-k's last step, finished where the entries are consumed.
// A query's selected set is its IN entries (certainly kept, in ascending
// order from the selection kernel) and the best rr = min(K - |IN|, |BAND|)
// band entries by (binary64 score descending, slot ascending).  The splits
// take positions 0 .. |IN| - 1 from the IN list and |IN| .. |IN| + rr - 1 from
// the chosen band entries in slot order; so only the blocks whose split
// reaches past |IN| (usually one per query) rank the band, and one block per
// query (the split holding position |IN|) writes the ascending index list:
// the IN bitmap with the chosen band bits set, compacted.  Nothing crosses
// blocks: everything comes from the earlier kernels' records.  `scr` is LDS
// scratch of `scr_words` words (the row buffer, before any row is staged).
template <int NT>
__device__ uint32_t att_block_sum(uint32_t v, uint32_t *red) {
    v = wave_sum_u32(v);
    __syncthreads();
    if ((threadIdx.x & 63) == 0) red[threadIdx.x >> 6] = v;
    __syncthreads();
    uint32_t t = 0;
#pragma unroll
    for (int i = 0; i < NT / 64; i++) t += red[i];
    return t;
}

// Band pick: the chosen band entries' bits in `bmb` (n / 32 words of LDS,
// zeroed here) and, for a block whose split reaches them, their entries in
// jsh (positions |IN| + rank in slot order).  `scr` (scr_words of LDS) holds
// the band's keys and slots while they are ranked.
template <int NT>
__device__ void att_sel_band(const SelHandoff &sel, int bq, int32_t in_cnt, int32_t nb, int32_t rr, int e_begin,
                             int ne, bool band_blk, int32_t spec_slot, double spec_score, uint32_t *bmb,
                             uint32_t *scr, int scr_words, int32_t *jsh, uint32_t *red) {
    const int tid = threadIdx.x;
    const int64_t n = sel.n;
    const int nw = (int)((n + 31) / 32);  // <= 1024 on this path
    const int32_t *list = sel.band + (size_t)bq * sel.band_cap;
    const double *bs = sel.band_score + (size_t)bq * sel.band_cap;
    const int32_t *cq = sel.cand ? sel.cand + (size_t)bq * n : nullptr;
    for (int w = tid; w < nw; w += NT) bmb[w] = 0u;
    const int cap = (scr_words - nw) / 4;  // entries; nw words after them for a tie group's bitmap
    u32x4 *ent = reinterpret_cast<u32x4 *>(scr);  // (key lo, key hi, slot, 0)
    if (nb <= cap) {
        // the first NT entries arrived with the block's first loads
        for (int32_t i = tid; i < nb; i += NT) {
            const int32_t sl = i == tid ? spec_slot : list[i];
            const uint64_t kk = dkey(i == tid ? spec_score : bs[i]);
            ent[i] = u32x4{(uint32_t)kk, (uint32_t)(kk >> 32), (uint32_t)sl, 0u};
        }
    }
    __syncthreads();
    if (nb <= cap) {
        // (key, slot) is ahead of entry i iff its key is larger, or equal
        // with a smaller slot.  First every entry counts the larger keys: a
        // wave takes 64 entries (one a lane) and 32 partners, loads the
        // partners' keys into 32 lanes and broadcasts each through scalar
        // registers, so a partner costs a compare and an add with carry,
        // unrolled, with no LDS latency.  The (entry chunk, partner chunk)
        // pairs are spread over the waves; keys past the end read as 0,
        // below every key of a finite score.  Entries with fewer than rr
        // larger keys are chosen: exactly rr of them unless the group of
        // equal keys at the cut straddles it.  That group is the chosen
        // entries with the most larger keys, G; then its first rr - G
        // members in slot order stay, found by a scan of its bitmap.
        constexpr int W = NT / 64, S = 32;
        __shared__ uint32_t n_chosen, g_cut;
        const int wave = __builtin_amdgcn_readfirstlane(tid >> 6), lane = tid & 63;
        const int C = (nb + 63) / 64, PC = (nb + S - 1) / S;
        if (tid == 0) n_chosen = 0, g_cut = 0;
        for (int task = wave; task < C * PC; task += W) {
            const int32_t i = (task / PC) * 64 + lane;
            const int32_t jl = (task % PC) * S + (lane & (S - 1));
            const bool act = i < nb;
            const u32x4 me = ent[act ? i : 0];
            const u32x4 o = ent[jl < nb ? jl : 0];
            const uint32_t plo = jl < nb ? o[0] : 0u, phi = jl < nb ? o[1] : 0u;
            const uint64_t ki = (uint64_t)me[0] | ((uint64_t)me[1] << 32);
            uint32_t gt = 0;
#pragma unroll
            for (int t = 0; t < S; t++) {
                const uint64_t kj = (uint64_t)(uint32_t)__builtin_amdgcn_readlane((int)plo, t) |
                                    ((uint64_t)(uint32_t)__builtin_amdgcn_readlane((int)phi, t) << 32);
                gt += kj > ki;
            }
            if (act) atomicAdd(reinterpret_cast<uint32_t *>(scr) + 4 * i + 3, gt);
        }
        __syncthreads();
        for (int32_t i0 = 0; i0 < nb; i0 += NT) {  // count and G: one LDS atomic per wave
            const int32_t i = i0 + tid;
            const u32x4 me = ent[i < nb ? i : 0];
            const bool ch = i < nb && me[3] < (uint32_t)rr;
            if (ch) atomicOr(&bmb[me[2] >> 5], 1u << (me[2] & 31));
            const uint32_t cnt = (uint32_t)__builtin_popcountll(__ballot(ch));
            const uint32_t gm = wave_max_u32(ch ? me[3] : 0u);
            if (lane == 0 && cnt) {
                atomicAdd(&n_chosen, cnt);
                atomicMax(&g_cut, gm);
            }
        }
        __syncthreads();
        if (n_chosen != (uint32_t)rr) {
            uint32_t *gb = scr + 4 * cap;  // the straddling group's bitmap (nw words)
            const uint32_t G = g_cut, need = (uint32_t)rr - G;
            for (int w = tid; w < nw; w += NT) gb[w] = 0u;
            __syncthreads();
            for (int32_t i = tid; i < nb; i += NT) {
                const u32x4 me = ent[i];
                if (me[3] == G) {
                    atomicOr(&gb[me[2] >> 5], 1u << (me[2] & 31));
                    atomicAnd(&bmb[me[2] >> 5], ~(1u << (me[2] & 31)));
                }
            }
            __syncthreads();
            const int per = (nw + NT - 1) / NT, w0 = tid * per;
            uint32_t c = 0;
            for (int w = w0; w < w0 + per && w < nw; w++) c += (uint32_t)__builtin_popcount(gb[w]);
            const uint32_t incl = wave_incl_scan_u32(c);
            if (lane == 63) red[wave] = incl;
            __syncthreads();
            uint32_t pos = incl - c;
#pragma unroll
            for (int q = 0; q < W; q++) pos += q < wave ? red[q] : 0u;
            for (int w = w0; w < w0 + per && w < nw; w++)
                for (uint32_t bb = gb[w]; bb && pos < need; bb &= bb - 1, pos++)
                    atomicOr(&bmb[w], 1u << __builtin_ctz(bb));
        }
    } else {
        // a band larger than the scratch: the rr-th best key by bisection
        // over the records, then the tie cut by slot
        uint64_t lo = 0, hi = ~0ull;  // largest key t with #(key >= t) >= rr
        while (lo < hi) {
            const uint64_t mid = lo + (hi - lo) / 2 + 1;
            uint32_t c = 0;
            for (int32_t i = tid; i < nb; i += NT) c += dkey(bs[i]) >= mid;
            if (att_block_sum<NT>(c, red) >= (uint32_t)rr) lo = mid;
            else hi = mid - 1;
        }
        const uint64_t tau = lo;
        uint32_t gt = 0;
        for (int32_t i = tid; i < nb; i += NT) gt += dkey(bs[i]) > tau;
        const uint32_t need = (uint32_t)rr - att_block_sum<NT>(gt, red);
        int64_t sl0 = 0, sl1 = n - 1;  // smallest slot cut with #(key == tau, slot <= cut) >= need
        while (sl0 < sl1) {
            const int64_t mid = sl0 + (sl1 - sl0) / 2;
            uint32_t c = 0;
            for (int32_t i = tid; i < nb; i += NT) c += dkey(bs[i]) == tau && list[i] <= mid;
            if (att_block_sum<NT>(c, red) >= need) sl1 = mid;
            else sl0 = mid + 1;
        }
        for (int32_t i = tid; i < nb; i += NT) {
            const uint64_t ki = dkey(bs[i]);
            const int32_t si = list[i];
            if (ki > tau || (ki == tau && si <= sl0 && need > 0)) atomicOr(&bmb[si >> 5], 1u << (si & 31));
        }
    }
    __syncthreads();
    if (band_blk) {
        // positions |IN| + (chosen entries before it in slot order); thread t owns words t * per ..
        const int per = (nw + NT - 1) / NT;
        const int w0 = tid * per;
        uint32_t c = 0;
        for (int w = w0; w < w0 + per && w < nw; w++) c += (uint32_t)__builtin_popcount(bmb[w]);
        const uint32_t incl = wave_incl_scan_u32(c);
        const int wave = tid >> 6, lane = tid & 63;
        if (lane == 63) red[wave] = incl;
        __syncthreads();
        uint32_t pos = (uint32_t)in_cnt + incl - c;
#pragma unroll
        for (int i = 0; i < NT / 64; i++) pos += i < wave ? red[i] : 0u;
        for (int w = w0; w < w0 + per && w < nw; w++)
            for (uint32_t bb = bmb[w]; bb; bb &= bb - 1) {
                const int32_t sl = w * 32 + __builtin_ctz(bb);
                if (pos >= (uint32_t)e_begin && pos < (uint32_t)(e_begin + ne)) jsh[pos - e_begin] = cq ? cq[sl] : sl;
                pos++;
            }
        __syncthreads();
    }
}

// The ascending index list of the query: the IN bitmap with the chosen band
// bits set (words `inw`, thread t holding words t * PW ..), compacted; -1 past
// the kept count.
template <int NT, int PW>
__device__ void att_sel_output(const SelHandoff &sel, int bq, int k, int32_t kept, const uint32_t (&inw)[PW],
                               uint32_t *red) {
    const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
    const int64_t n = sel.n;
    const int nw = (int)((n + 31) / 32);
    const int w0 = tid * PW;
    const int32_t *cq = sel.cand ? sel.cand + (size_t)bq * n : nullptr;
    uint32_t bits[PW], c = 0;
#pragma unroll
    for (int u = 0; u < PW; u++) {
        bits[u] = w0 + u < nw ? inw[u] : 0u;
        c += (uint32_t)__builtin_popcount(bits[u]);
    }
    const uint32_t incl = wave_incl_scan_u32(c);
    if (lane == 63) red[wave] = incl;
    __syncthreads();
    uint32_t pos = incl - c;
#pragma unroll
    for (int i = 0; i < NT / 64; i++) pos += i < wave ? red[i] : 0u;
    int32_t *orow = sel.idx + (size_t)bq * k;
#pragma unroll
    for (int u = 0; u < PW; u++)
        for (uint32_t bb = bits[u]; bb; bb &= bb - 1) {
            if (pos < (uint32_t)k) {
                const int32_t sl = (w0 + u) * 32 + __builtin_ctz(bb);
                orow[pos] = cq ? cq[sl] : sl;
            }
            pos++;
        }
    for (int32_t i = kept + tid; i < k; i += NT) orow[i] = -1;
    if (tid == 0 && sel.count) sel.count[bq] = kept;
    __syncthreads();
}

// ------------------------------------------------------- split kernel
// Block = one query x one split of ATT_SPLIT = 128 selected entries x HB =
// HPW * HH heads, 4 HH waves.  The LDS read traffic per gathered row is what
// bounds this step (S and O read every row from LDS), so the block is laid
// out to read each row as few times as the registers allow:
//  1. Every row of the split is requested at once (16-byte pieces in
//     registers, one wave per 1 KiB of a bf16 row), then staged in LDS as the
//     matrix-core operand type (FP4 rows decoded to fp16 on the way).
//  2. S^T = C Q^T: wave (rg, hh) takes rows 32 rg .. 32 rg + 31 and heads
//     hh HPW .. + HPW - 1 over all D channels, its queries held in registers
//     for the whole contraction; each row fragment read from LDS feeds HPW/16
//     matrix-core steps.  No partial logits cross waves.
//  3. Softmax over the split: each head's maximum over the four row groups
//     meets in LDS; p = exp(a - m) goes to LDS as P[head][row] (the
//     matrix-core operand type), each row group's sum of p to LDS.
//  4. O^T = C^T P^T: wave (cq, hh) takes channels cq D/4 .. + D/4 - 1 of the
//     same heads; the row operand is read transposed from the staged rows,
//     P^T from LDS; 32 rows per step, in row order.
//  5. Output (one split: out / l, lse) or the split partial (fp16 under a
//     power-of-two scale per head and quarter of the channels, m, l) for the
//     merge kernel.
// Every head's arithmetic (contraction order over channels and rows, the
// sums of p over rows grouped by 32, the fixed tree over the four groups) is
// the same whatever HB, so a query's result does not depend on the batch.
template <int D, int FMT, int HPW, int HH, bool SEL>
__global__ __launch_bounds__(256 * HH, 1) void k_attn_split(const uint16_t *__restrict__ q,
                                                           const uint8_t *__restrict__ kv, int Q, int H, int64_t N,
                                                           const int32_t *__restrict__ idx, int k, float scale,
                                                           int nsplit, int npairs, uint16_t *__restrict__ out,
                                                           float *__restrict__ lse, uint16_t *__restrict__ part_o,
                                                           float2 *__restrict__ part_ml, float *__restrict__ part_sc,
                                                           SelHandoff sel) {
    constexpr int NW = 4 * HH, NT = 64 * NW;
    constexpr int HB = HPW * HH;      // heads of the block
    constexpr int HT = HPW / 16;      // 16-head tiles of a wave
    constexpr int KS = D / 32;        // contraction steps of S (32 channels each)
    constexpr int LS = D + 8;         // LDS row stride in 16-bit elements (16-byte pad)
    constexpr int ROWS = ATT_SPLIT;   // entries of a split
    constexpr int PST = ROWS + 8;     // LDS stride of a head's P row
    constexpr int DQ = D / 4;         // channels of an O wave (one quarter)
    constexpr int DT = DQ / 16;       // 16-channel tiles of an O wave
    constexpr int KT = ROWS / 32;     // contraction steps of O (32 rows each)
    constexpr int RB = FMT == CSA2_FP4 ? D / 2 + D / 16 : 2 * D;  // bytes per stored row
    static_assert(DQ % 16 == 0 && HPW % 16 == 0, "matrix-core tiles");
    __shared__ __attribute__((aligned(16))) uint16_t rows_lds[ROWS * LS];
    __shared__ __attribute__((aligned(16))) uint16_t p_lds[HB * PST];
    __shared__ float mx_sh[4][HB];
    __shared__ float l_sh[4][HB];
    __shared__ float qsc_sh[HB];  // FP4: softmax scale times the head's query prescale
    __shared__ __attribute__((aligned(16))) int32_t jsh[ROWS];

    // Blocks go round-robin over the 8 XCDs (block L to XCD L % 8): XCD x
    // takes the consecutive (query, split) pairs x P8 .. x P8 + P8 - 1, so that
    // the blocks of a query share one L2 for its queries and, across head
    // groups, for its rows.
    const int NG = H / HB;
    const int P8 = (npairs + 7) / 8;
    const int L = blockIdx.x;
    const int jx = (L / 8) / NG;
    const int hgb = (L / 8) % NG;
    const int pair = (L % 8) * P8 + jx;
    if (jx >= P8 || pair >= npairs) return;
    const int split = pair % nsplit;
    const int bq = pair / nsplit;
    const int b = bq / Q;
    const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
    const int col = lane & 15, kg = lane >> 4;
    const int rq = wave & 3;   // row group (S) and channel quarter (O) of this wave
    const int hh = wave >> 2;  // head half of the block
    const int hw0 = hh * HPW;  // first head of this wave within the block
    const int e_begin = split * ROWS;
    const int ne = min(k, e_begin + ROWS) - e_begin;
    const uint8_t *kvb = kv + (size_t)b * N * RB;

    // the block's query heads first: they do not depend on the indices.  Not
    // so in the last split with a selection to finish, which usually ranks
    // the band: its LDS work would wait behind these loads, so there they
    // are issued after the ranking, still ahead of the rows.
    constexpr int QS = D + 8;
    constexpr int QPR = D / 8;                 // 16-byte pieces per head row
    constexpr int QP = HB * QPR;
    constexpr int QPT = (QP + NT - 1) / NT;
    u32x4 qst[QPT];
    const bool q_early = !SEL || split != nsplit - 1;
    auto load_q = [&]() {
        const u32x4 *qsrc = reinterpret_cast<const u32x4 *>(q + ((size_t)bq * H + hgb * HB) * D);
#pragma unroll
        for (int i = 0; i < QPT; i++) qst[i] = qsrc[QP % NT == 0 ? tid + NT * i : min(tid + NT * i, QP - 1)];
    };
    if (q_early) load_q();
    // certified selection finished here (SEL): the query's IN count, band size
    // and chosen band count; the block that writes the index list keeps its
    // IN bitmap words (loaded with everything else, before any wait)
    __shared__ uint32_t sred[NT / 64];
    constexpr int SPW = (1024 + NT - 1) / NT;  // IN bitmap words per thread (n <= 32768)
    uint32_t inw[SPW];
    int32_t in_cnt = 0, rr = 0;
    bool out_blk = false;
    if constexpr (SEL) {
        // speculative: the last split usually holds the band's part of the set,
        // so it loads the first NT band records with the target record
        const bool spec = split == nsplit - 1;
        const size_t bo = (size_t)bq * sel.band_cap + (tid < sel.band_cap ? tid : 0);
        const int32_t spec_slot = spec ? sel.band[bo] : 0;
        const double spec_score = spec ? sel.band_score[bo] : 0.0;
        const SelTarget t = sel.sq[bq].t[0];
        in_cnt = t.in_cnt;
        const int32_t nb = t.band_cnt;
        rr = max(0, min(k - in_cnt, nb));
        out_blk = hgb == 0 && split == min(in_cnt, k - 1) / ROWS;
        const int nw = (int)sel.nwords;
        const uint32_t *inbm = sel.bitmap + (size_t)bq * sel.nwords;
#pragma unroll
        for (int u = 0; u < SPW; u++) inw[u] = (out_blk && tid * SPW + u < nw) ? inbm[tid * SPW + u] : 0u;
        const int32_t *il = sel.in_list + (size_t)bq * sel.in_cap;
        for (int e = tid; e < ROWS; e += NT) {
            const int p = e_begin + e;
            jsh[e] = (e < ne && p < in_cnt) ? il[p] : -1;
        }
        const bool band_blk = rr > 0 && e_begin + ne > in_cnt;
        if (band_blk || (out_blk && rr > 0)) {
            const bool have = spec && tid < sel.band_cap;
            att_sel_band<NT>(sel, bq, in_cnt, nb, rr, e_begin, ne, band_blk,
                             have ? spec_slot : sel.band[bo], have ? spec_score : sel.band_score[bo],
                             reinterpret_cast<uint32_t *>(p_lds), reinterpret_cast<uint32_t *>(rows_lds),
                             ROWS * LS / 2, jsh, sred);
        }
        else if (out_blk)
            for (int w = tid; w < nw; w += NT) reinterpret_cast<uint32_t *>(p_lds)[w] = 0u;
    } else {
        const int32_t *irow = idx + (size_t)bq * k + e_begin;
        for (int e = tid; e < ROWS; e += NT) {
            const int j = e < ne ? irow[e] : -1;
            jsh[e] = (j >= 0 && j < N) ? j : -1;  // out-of-range entries are skipped like -1
        }
    }
    __syncthreads();

    // ---- 1. gather.  bf16: piece c = 16 bytes (8 channels) of row c / CPR at
    // column c % CPR, a wave reads one whole 1 KiB row per instruction.  FP4:
    // piece c = 4 code bytes (8 channels) and their scale byte, a wave reads one
    // row's 256 code bytes per instruction; decoded to 16 bytes of fp16.
    // Either way lane l writes 16 bytes at column l of a row: no LDS bank
    // conflicts.  Entries of -1 read row 0 and are zeroed.
    constexpr int PPR = D / 8;                 // 8-channel pieces per row
    constexpr int NPC = ROWS * PPR;            // pieces of the split
    constexpr int PPT = (NPC + NT - 1) / NT;  // pieces per thread
    constexpr int GR = PPT > 16 ? 16 : PPT;    // pieces per thread in flight
    static_assert(PPT % GR == 0, "whole rounds of pieces");
    uint32_t gw[FMT == CSA2_FP4 ? GR : 1];     // FP4: code word
    u32x4 gv[FMT == CSA2_FP4 ? 1 : GR];        // bf16: 16 bytes
    uint32_t gs[GR];                           // FP4 scale byte | no-entry flag in bit 31
    auto issue = [&](int r0) {
#pragma unroll
        for (int u = 0; u < GR; u++) {
            const int c = tid + (r0 + u) * NT;
            const int cs = (NPC % NT == 0 || c < NPC) ? c : 0;
            const int r = cs / PPR, cc = cs % PPR;
            const int j = jsh[r];
            const uint8_t *row = kvb + (size_t)(j >= 0 ? j : 0) * RB;
            uint32_t sc = 0;
            if constexpr (FMT == CSA2_FP4) {
                gw[u] = *reinterpret_cast<const uint32_t *>(row + cc * 4);
                sc = row[D / 2 + cc / 2];
            } else {
                gv[u] = *reinterpret_cast<const u32x4 *>(row + cc * 16);
            }
            gs[u] = sc | (j < 0 ? 0x80000000u : 0u);
        }
    };
    auto store = [&](int r0) {
#pragma unroll
        for (int u = 0; u < GR; u++) {
            const int c = tid + (r0 + u) * NT;
            if (NPC % NT != 0 && c >= NPC) continue;
            const int r = c / PPR, cc = c % PPR;
            const bool skip = gs[u] >> 31;
            u32x4 v;
            if constexpr (FMT == CSA2_FP4) v = fp4_word_to_f16x8(skip ? 0u : gw[u], skip ? 0u : gs[u] & 0xffu);
            else v = skip ? u32x4{0u, 0u, 0u, 0u} : gv[u];
            *reinterpret_cast<u32x4 *>(rows_lds + r * LS + cc * 8) = v;
        }
    };
    if constexpr (SEL) {
        // the chosen band bits join the output block's IN words in registers
        // (P's LDS is reused by the softmax); the list is written at the end
        if (out_blk) {
            const int nw = (int)sel.nwords;
#pragma unroll
            for (int u = 0; u < SPW; u++)
                if (tid * SPW + u < nw) inw[u] |= reinterpret_cast<const uint32_t *>(p_lds)[tid * SPW + u];
        }
    }
    if (!q_early) load_q();
    issue(0);
    __builtin_amdgcn_sched_barrier(0);

    // ---- the block's query heads, once per block (each is the B operand of
    // S^T for four waves): in flight from the start, staged in the row buffer
    // (padded rows of D + 8) before the rows land; for FP4 rows converted to
    // fp16 there under a power-of-two scale per head that keeps them below
    // 32768 (a wave holds whole head rows: piece i of thread t is 16 bytes of
    // head (t + NT i) / (D / 8))
    static_assert(HB * QS <= ROWS * LS, "query staging fits the row buffer");
    static_assert(QPR <= 64 && 64 % QPR == 0, "a head's query row lies within one wave");
    {
#pragma unroll
        for (int i = 0; i < QPT; i++) {
            const int pc = tid + NT * i;
            const int hq = pc / QPR, cq = pc % QPR;
            u32x4 v = qst[i];
            if constexpr (FMT == CSA2_FP4) {
                float amax = 0.f;
#pragma unroll
                for (int e = 0; e < 4; e++)
                    amax = fmaxf(amax, fmaxf(fabsf(bf16_to_f32(v[e] & 0xffffu)), fabsf(bf16_to_f32(v[e] >> 16))));
                // the QPR consecutive lanes holding the head's row
                if constexpr (QPR == 64) {
                    amax = wave_max(amax);
                } else {
#pragma unroll
                    for (int o = 1; o < QPR; o <<= 1) amax = fmaxf(amax, __shfl_xor(amax, o));
                }
                int ex = 0;
                if (amax > 32768.f) ex = (int)ceilf(log2f(amax / 32768.f));
                const float down = ldexpf(1.f, -ex);
                if (cq == 0 && (QP % NT == 0 || pc < QP)) qsc_sh[hq] = ldexpf(scale, ex);
#pragma unroll
                for (int e = 0; e < 4; e++)
                    v[e] = pack_f16_rne(bf16_to_f32(v[e] & 0xffffu) * down, bf16_to_f32(v[e] >> 16) * down);
            }
            if (QP % NT == 0 || pc < QP) *reinterpret_cast<u32x4 *>(rows_lds + hq * QS + cq * 8) = v;
        }
    }
    __syncthreads();
    u32x4 qf[HT][KS];
#pragma unroll
    for (int ht = 0; ht < HT; ht++)
#pragma unroll
        for (int s2 = 0; s2 < KS; s2++)
            qf[ht][s2] = *reinterpret_cast<const u32x4 *>(rows_lds + (hw0 + 16 * ht + col) * QS + 32 * s2 + 8 * kg);
    float qscale[HT];
#pragma unroll
    for (int ht = 0; ht < HT; ht++) qscale[ht] = FMT == CSA2_FP4 ? qsc_sh[hw0 + 16 * ht + col] : scale;
    __syncthreads();  // the row buffer is free again

    store(0);
#pragma unroll
    for (int r0 = GR; r0 < PPT; r0 += GR) {
        issue(r0);
        store(r0);
    }
    __syncthreads();  // rows staged

    // ---- 2. S^T for rows 32 rq + 16 h2 + (lane rows), heads hw0 + 16 ht + col
    f32x4 sacc[2][HT];
#pragma unroll
    for (int h2 = 0; h2 < 2; h2++)
#pragma unroll
        for (int ht = 0; ht < HT; ht++) sacc[h2][ht] = f32x4{0.f, 0.f, 0.f, 0.f};
    {
        const uint16_t *arow = rows_lds + (32 * rq + col) * LS + 8 * kg;
#pragma unroll
        for (int s2 = 0; s2 < KS; s2++) {
            const u32x4 a0 = *reinterpret_cast<const u32x4 *>(arow + 32 * s2);
            const u32x4 a1 = *reinterpret_cast<const u32x4 *>(arow + 16 * LS + 32 * s2);
#pragma unroll
            for (int ht = 0; ht < HT; ht++) {
                sacc[0][ht] = mma<FMT>(a0, qf[ht][s2], sacc[0][ht]);
                sacc[1][ht] = mma<FMT>(a1, qf[ht][s2], sacc[1][ht]);
            }
        }
    }
    // ---- 3. softmax over the split. Lane holds rows 32 rq + 16 h2 + 4 kg + i.
    const int4 jv0 = *reinterpret_cast<const int4 *>(jsh + 32 * rq + 4 * kg);
    const int4 jv1 = *reinterpret_cast<const int4 *>(jsh + 32 * rq + 16 + 4 * kg);
    const int jj[8] = {jv0.x, jv0.y, jv0.z, jv0.w, jv1.x, jv1.y, jv1.z, jv1.w};
    float mloc[HT];
#pragma unroll
    for (int ht = 0; ht < HT; ht++) {
        float mt = NEG_INF;
#pragma unroll
        for (int x = 0; x < 8; x++) {
            const float v = jj[x] >= 0 ? sacc[x >> 2][ht][x & 3] * qscale[ht] : NEG_INF;
            sacc[x >> 2][ht][x & 3] = v;
            mt = fmaxf(mt, v);
        }
        mloc[ht] = bfly32(bfly16(mt, OpMax{}), OpMax{});
        if (kg == 0) mx_sh[rq][hw0 + 16 * ht + col] = mloc[ht];
    }
    __syncthreads();
    float mh[HT];
#pragma unroll
    for (int ht = 0; ht < HT; ht++) {
        const int hd = hw0 + 16 * ht + col;
        mh[ht] = fmaxf(fmaxf(mx_sh[0][hd], mx_sh[1][hd]), fmaxf(mx_sh[2][hd], mx_sh[3][hd]));
        float ls = 0.f;
#pragma unroll
        for (int h2 = 0; h2 < 2; h2++) {
            float pv[4];
#pragma unroll
            for (int i = 0; i < 4; i++) {
                const float a = sacc[h2][ht][i];
                pv[i] = a == NEG_INF ? 0.f : __expf(a - mh[ht]);
                ls += pv[i];
            }
            uint32_t w0, w1;
            if constexpr (FMT == CSA2_FP4) {
                w0 = pack_f16_rne(pv[0], pv[1]);
                w1 = pack_f16_rne(pv[2], pv[3]);
            } else {
                w0 = __builtin_bit_cast(uint32_t, __builtin_convertvector((f32x2{pv[0], pv[1]}), bf16x2v));
                w1 = __builtin_bit_cast(uint32_t, __builtin_convertvector((f32x2{pv[2], pv[3]}), bf16x2v));
            }
            *reinterpret_cast<uint2 *>(p_lds + hd * PST + 32 * rq + 16 * h2 + 4 * kg) = make_uint2(w0, w1);
        }
        ls = bfly32(bfly16(ls, OpAdd{}), OpAdd{});
        if (kg == 0) l_sh[rq][hd] = ls;
    }
    __syncthreads();

    // ---- 4. O^T[channel][head] for channels rq DQ + 16 dt + (lane rows), heads hw0 + 16 ht + col
    f32x4 oacc[DT][HT];
#pragma unroll
    for (int dt = 0; dt < DT; dt++)
#pragma unroll
        for (int ht = 0; ht < HT; ht++) oacc[dt][ht] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int kt = 0; kt < KT; kt++) {
        // operand element x <-> row 32 kt + 16 (x / 4) + 4 kg + x % 4, in both operands
        u32x4 pb[HT];
#pragma unroll
        for (int ht = 0; ht < HT; ht++) {
            const uint16_t *pp = p_lds + (hw0 + 16 * ht + col) * PST + 32 * kt + 4 * kg;
            const uint2 lo = *reinterpret_cast<const uint2 *>(pp);
            const uint2 hi = *reinterpret_cast<const uint2 *>(pp + 16);
            pb[ht] = u32x4{lo.x, lo.y, hi.x, hi.y};
        }
        const uint16_t *tr0 = rows_lds + (32 * kt + 4 * kg + (col >> 2)) * LS + 4 * (col & 3) + rq * DQ;
        const uint16_t *tr1 = tr0 + 16 * LS;
#pragma unroll
        for (int dt = 0; dt < DT; dt++) {
            const s16x4 lo4 = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
                (s16x4 __attribute__((address_space(3))) *)(tr0 + 16 * dt));
            const s16x4 hi4 = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
                (s16x4 __attribute__((address_space(3))) *)(tr1 + 16 * dt));
            const u32x4 av = {__builtin_bit_cast(uint32_t, s16x2{lo4[0], lo4[1]}),
                              __builtin_bit_cast(uint32_t, s16x2{lo4[2], lo4[3]}),
                              __builtin_bit_cast(uint32_t, s16x2{hi4[0], hi4[1]}),
                              __builtin_bit_cast(uint32_t, s16x2{hi4[2], hi4[3]})};
#pragma unroll
            for (int ht = 0; ht < HT; ht++) oacc[dt][ht] = mma<FMT>(av, pb[ht], oacc[dt][ht]);
        }
    }

    // ---- 5. output (one split: out / l, lse) or the split partial (fp16
    // under a power-of-two scale per head and channel quarter, m, l), staged
    // in the free row buffer as [head][channel] so that the block writes its
    // HB consecutive rows of D in whole 16-byte pieces per lane
    __syncthreads();  // every wave is done with the rows
    constexpr int OS = D + 8;
    uint16_t *stage = rows_lds;
#pragma unroll
    for (int ht = 0; ht < HT; ht++) {
        const int hd = hw0 + 16 * ht + col;
        const int h = hgb * HB + hd;
        const float l = (l_sh[0][hd] + l_sh[1][hd]) + (l_sh[2][hd] + l_sh[3][hd]);
        const float m = mh[ht];
        uint16_t *srow = stage + hd * OS + rq * DQ + 4 * kg;
        if (nsplit == 1) {
            const float inv = l > 0.f ? 1.f / l : 0.f;
#pragma unroll
            for (int dt = 0; dt < DT; dt++) {
                const f32x4 o = oacc[dt][ht];
                const uint32_t w0 = uint32_t(f32_to_bf16_rne(o[0] * inv)) | (uint32_t(f32_to_bf16_rne(o[1] * inv)) << 16);
                const uint32_t w1 = uint32_t(f32_to_bf16_rne(o[2] * inv)) | (uint32_t(f32_to_bf16_rne(o[3] * inv)) << 16);
                *reinterpret_cast<uint2 *>(srow + 16 * dt) = make_uint2(w0, w1);
            }
            if (lse && kg == 0 && rq == 0) lse[(size_t)bq * H + h] = l > 0.f ? m + logf(l) : NEG_INF;
        } else {
            const size_t pi = ((size_t)bq * nsplit + split) * H + h;
            float mx = 0.f;
#pragma unroll
            for (int dt = 0; dt < DT; dt++)
#pragma unroll
                for (int r = 0; r < 4; r++) mx = fmaxf(mx, fabsf(oacc[dt][ht][r]));
            mx = bfly32(bfly16(mx, OpMax{}), OpMax{});
            // ex with mx in [2^(ex+14), 2^(ex+15)), from the exponent field,
            // clamped to [-120, 120] (subnormal maxima take -120; zero and
            // non-finite ones 0)
            const int ef = (int)((__float_as_uint(mx) >> 23) & 0xffu);
            const int ex = ef == 255 ? 0 : ef == 0 ? (mx > 0.f ? -120 : 0) : min(max(ef - 126 - 15, -120), 120);
            const float down = __uint_as_float((uint32_t)(127 - ex) << 23);
#pragma unroll
            for (int dt = 0; dt < DT; dt++) {
                const f32x4 o = oacc[dt][ht];
                *reinterpret_cast<uint2 *>(srow + 16 * dt) =
                    make_uint2(pack_f16_rne(o[0] * down, o[1] * down), pack_f16_rne(o[2] * down, o[3] * down));
            }
            if (kg == 0) part_sc[pi * 4 + rq] = __uint_as_float((uint32_t)(127 + ex) << 23);
            if (kg == 0 && rq == 0) part_ml[pi] = make_float2(m, l);
        }
    }
    __syncthreads();
    {
        uint16_t *dst = nsplit == 1 ? out + ((size_t)bq * H + hgb * HB) * D
                                    : part_o + (((size_t)bq * nsplit + split) * H + hgb * HB) * D;
        constexpr int OP = HB * D / 8;  // 16-byte pieces of the block's rows
#pragma unroll
        for (int i = tid; i < OP; i += NT) {
            const int r = i / (D / 8), c = i % (D / 8);
            *reinterpret_cast<u32x4 *>(dst + (size_t)r * D + 8 * c) =
                *reinterpret_cast<const u32x4 *>(stage + r * OS + 8 * c);
        }
    }
    // the query's ascending index list (SEL: the block holding position |IN|),
    // last, so that its stores do not stand in the loads' way
    if constexpr (SEL) {
        if (out_blk) att_sel_output<NT, SPW>(sel, bq, k, in_cnt + rr, inw, sred);
    }
}

// ------------------------------------------------------- prefill kernel
// Block = one query token x HB = HPW * HH heads, over all k of its selected
// entries in tiles of 64 rows: a prefill chunk has thousands of queries, so
// whole queries fill the chip and no split partials go through memory.  The
// rows of tile t + 1 are copied straight from HBM into the second LDS buffer
// (16-byte global->LDS loads, one 1 KiB row per wave instruction, no
// registers) while tile t is computed from the first, and the softmax runs
// online: each tile's maximum per head joins the running one, which rescales
// the running sum and the O^T accumulators before the tile's P C is added.
// Phases per tile, as in the split kernel: S^T = C Q^T (wave (rq, hh): rows
// 16 rq .. 16 rq + 15, heads hh HPW ..), p = exp(a - m) to LDS, O^T = C^T P^T
// (wave (rq, hh): channels rq D/4 ..).  bf16 rows of D = 512 only (a row is one
// wave-wide load).  A query's result does not depend on B, Q or the batch.
constexpr int TROWS = 64;

// 16 bytes per lane from global memory straight into LDS: lane l's bytes land
// at dst + 16 l (dst is the same for the whole wave).  A device function of
// its own, so that the host side of the kernel never sees the builtin.
__device__ __forceinline__ void copy16_to_lds(const uint16_t *src, uint16_t *dst) {
    __builtin_amdgcn_global_load_lds(src, dst, 16, 0, 0);
}

// A block barrier that orders the block's own LDS reads and writes only:
// __syncthreads() is a workgroup fence, which also waits for the global->LDS
// row copies still in flight (they count as LDS writes), so a barrier in the
// middle of a tile would wait for the next tile's rows.
__device__ __forceinline__ void lds_barrier() { asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory"); }

template <int D, int HPW, int HH>
__global__ __launch_bounds__(256 * HH, 1) void k_attn_tiles(const uint16_t *__restrict__ q,
                                                           const uint16_t *__restrict__ kv, int Q, int H, int64_t N,
                                                           const int32_t *__restrict__ idx, int k, float scale,
                                                           int nq, uint16_t *__restrict__ out, float *__restrict__ lse) {
    constexpr int NW = 4 * HH, NT = 64 * NW;
    constexpr int HB = HPW * HH;
    constexpr int HT = HPW / 16;
    constexpr int KS = D / 32;
    constexpr int LS = D + 8;          // LDS row stride (16-bit elements)
    constexpr int DQ = D / 4;
    constexpr int DT = DQ / 16;
    constexpr int KT = TROWS / 32;     // O contraction steps per tile
    constexpr int PST = TROWS + 8;     // P row stride
    constexpr int QS = D + 8;
    static_assert(D == 512, "one bf16 row is one 64-lane load of 16 bytes");
    static_assert(HB * QS <= TROWS * LS, "query staging fits a row buffer");
    // two row buffers (and entry lists) as separate LDS variables, each named
    // statically below: the compiler then knows that reading one does not
    // alias the global->LDS copies in flight into the other, and does not wait
    // for them (with one array indexed by the tile's parity it waited for the
    // next tile's rows before every tile)
    __shared__ __attribute__((aligned(16))) uint16_t rows_a[TROWS * LS];
    __shared__ __attribute__((aligned(16))) uint16_t rows_b[TROWS * LS];
    __shared__ __attribute__((aligned(16))) uint16_t p_lds[HB * PST];
    __shared__ float mx_sh[4][HB];
    __shared__ float l_sh[4][HB];
    __shared__ __attribute__((aligned(16))) int32_t jsh_a[TROWS];
    __shared__ __attribute__((aligned(16))) int32_t jsh_b[TROWS];

    // block L on XCD L % 8: consecutive queries (which share most of their
    // rows) on one XCD, the head groups of a query beside them
    const int NG = H / HB;
    const int P8 = (nq + 7) / 8;
    const int L = blockIdx.x;
    const int jx = (L / 8) / NG;
    const int hgb = (L / 8) % NG;
    const int bq = (L % 8) * P8 + jx;
    if (jx >= P8 || bq >= nq) return;
    const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
    const int col = lane & 15, kg = lane >> 4;
    const int rq = wave & 3, hh = wave >> 2, hw0 = hh * HPW;
    const int ntl = (k + TROWS - 1) / TROWS;
    const int32_t *irow = idx + (size_t)bq * k;
    const uint16_t *kvb = kv + (size_t)(bq / Q) * N * D;

    // ---- query heads: registers -> LDS [head][QS] -> this wave's fragments
    constexpr int QP = HB * D / 8, QPT = (QP + NT - 1) / NT;
    {
        const u32x4 *qsrc = reinterpret_cast<const u32x4 *>(q + ((size_t)bq * H + hgb * HB) * D);
        u32x4 qst[QPT];
#pragma unroll
        for (int i = 0; i < QPT; i++) qst[i] = qsrc[QP % NT == 0 ? tid + NT * i : min(tid + NT * i, QP - 1)];
        uint16_t *qs = rows_a;
#pragma unroll
        for (int i = 0; i < QPT; i++) {
            const int pc = tid + NT * i;
            if (QP % NT == 0 || pc < QP) *reinterpret_cast<u32x4 *>(qs + (pc / (D / 8)) * QS + (pc % (D / 8)) * 8) = qst[i];
        }
    }
    for (int e = tid; e < TROWS; e += NT) {
        const int j = e < k ? irow[e] : -1;
        jsh_a[e] = (j >= 0 && j < N) ? j : -1;
    }
    __syncthreads();
    u32x4 qf[HT][KS];
#pragma unroll
    for (int ht = 0; ht < HT; ht++)
#pragma unroll
        for (int s2 = 0; s2 < KS; s2++)
            qf[ht][s2] = *reinterpret_cast<const u32x4 *>(rows_a + (hw0 + 16 * ht + col) * QS + 32 * s2 + 8 * kg);
    __syncthreads();  // the row buffers are free

    // rows of a tile into buffer dst: wave w copies rows w, w + NW, ...; an
    // entry of -1 copies row 0 (masked later)
    auto issue = [&](uint16_t *dst, const int32_t *js) {
#pragma unroll
        for (int r = wave; r < TROWS; r += NW) {
            const int j = __builtin_amdgcn_readfirstlane(js[r]);
            const uint16_t *src = kvb + (size_t)(j >= 0 ? j : 0) * D + 8 * lane;
            copy16_to_lds(src, dst + r * LS);
        }
    };
    issue(rows_a, jsh_a);
    // next tile's entry of this thread (tid < TROWS), as loaded: range-checked
    // only when it goes to LDS after the tile's wait, so that checking it does
    // not wait for the row copies issued before it
    int jn = -1;
    if (tid < TROWS && TROWS + tid < k) jn = irow[TROWS + tid];

    f32x4 oacc[DT][HT];
#pragma unroll
    for (int dt = 0; dt < DT; dt++)
#pragma unroll
        for (int ht = 0; ht < HT; ht++) oacc[dt][ht] = f32x4{0.f, 0.f, 0.f, 0.f};
    float m_run[HT], l_run[HT];
#pragma unroll
    for (int ht = 0; ht < HT; ht++) {
        m_run[ht] = NEG_INF;
        l_run[ht] = 0.f;
    }

    // tile t from rows / jcur while tile t + 1 is copied into nrows / jnext
    auto step = [&](int t, const uint16_t *__restrict__ rows, const int32_t *__restrict__ jcur,
                    uint16_t *__restrict__ nrows, int32_t *__restrict__ jnext) __attribute__((always_inline)) {
        // this tile's rows (and the next tile's entries) have landed
        asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
        if (tid < TROWS) jnext[tid] = (jn >= 0 && jn < N) ? jn : -1;
        __syncthreads();
        if (t + 1 < ntl) {
            issue(nrows, jnext);
            jn = -1;
            const int e = (t + 2) * TROWS + tid;
            if (tid < TROWS && e < k) jn = irow[e];
        }

        // S^T for rows 16 rq + 4 kg + i, heads hw0 + 16 ht + col
        f32x4 sacc[HT];
#pragma unroll
        for (int ht = 0; ht < HT; ht++) sacc[ht] = f32x4{0.f, 0.f, 0.f, 0.f};
        {
            const uint16_t *arow = rows + (16 * rq + col) * LS + 8 * kg;
#pragma unroll
            for (int s2 = 0; s2 < KS; s2++) {
                const u32x4 a0 = *reinterpret_cast<const u32x4 *>(arow + 32 * s2);
#pragma unroll
                for (int ht = 0; ht < HT; ht++) sacc[ht] = mma<CSA2_BF16>(a0, qf[ht][s2], sacc[ht]);
            }
        }
        const int4 jv = *reinterpret_cast<const int4 *>(&jcur[16 * rq + 4 * kg]);
        const int jj[4] = {jv.x, jv.y, jv.z, jv.w};
#pragma unroll
        for (int ht = 0; ht < HT; ht++) {
            float mt = NEG_INF;
#pragma unroll
            for (int i = 0; i < 4; i++) {
                const float v = jj[i] >= 0 ? sacc[ht][i] * scale : NEG_INF;
                sacc[ht][i] = v;
                mt = fmaxf(mt, v);
            }
            mt = bfly32(bfly16(mt, OpMax{}), OpMax{});
            if (kg == 0) mx_sh[rq][hw0 + 16 * ht + col] = mt;
        }
        lds_barrier();
        float alpha[HT];
#pragma unroll
        for (int ht = 0; ht < HT; ht++) {
            const int hd = hw0 + 16 * ht + col;
            const float mt = fmaxf(fmaxf(mx_sh[0][hd], mx_sh[1][hd]), fmaxf(mx_sh[2][hd], mx_sh[3][hd]));
            const float mh = fmaxf(m_run[ht], mt);
            alpha[ht] = mh == NEG_INF ? 1.f : (m_run[ht] == NEG_INF ? 0.f : __expf(m_run[ht] - mh));
            m_run[ht] = mh;
            float pv[4], ls = 0.f;
#pragma unroll
            for (int i = 0; i < 4; i++) {
                const float a = sacc[ht][i];
                pv[i] = a == NEG_INF ? 0.f : __expf(a - mh);
                ls += pv[i];
            }
            const uint32_t w0 = __builtin_bit_cast(uint32_t, __builtin_convertvector((f32x2{pv[0], pv[1]}), bf16x2v));
            const uint32_t w1 = __builtin_bit_cast(uint32_t, __builtin_convertvector((f32x2{pv[2], pv[3]}), bf16x2v));
            *reinterpret_cast<uint2 *>(p_lds + hd * PST + 16 * rq + 4 * kg) = make_uint2(w0, w1);
            ls = bfly32(bfly16(ls, OpAdd{}), OpAdd{});
            if (kg == 0) l_sh[rq][hd] = ls;
        }
        lds_barrier();
        // O^T[channel][head] += C^T P^T for channels rq DQ + 16 dt + (lane rows)
        // (the accumulators are rescaled only when some head's maximum moved:
        // after the first tiles that is rare, and multiplying by 1 is exact)
        bool moved = false;
#pragma unroll
        for (int ht = 0; ht < HT; ht++) {
            const int hd = hw0 + 16 * ht + col;
            l_run[ht] = l_run[ht] * alpha[ht] + ((l_sh[0][hd] + l_sh[1][hd]) + (l_sh[2][hd] + l_sh[3][hd]));
            moved |= alpha[ht] != 1.f;
        }
        if (__builtin_amdgcn_ballot_w64(moved)) {
#pragma unroll
            for (int ht = 0; ht < HT; ht++)
#pragma unroll
                for (int dt = 0; dt < DT; dt++)
#pragma unroll
                    for (int r = 0; r < 4; r++) oacc[dt][ht][r] *= alpha[ht];
        }
#pragma unroll
        for (int kt = 0; kt < KT; kt++) {
            u32x4 pb[HT];
#pragma unroll
            for (int ht = 0; ht < HT; ht++) {
                const uint16_t *pp = p_lds + (hw0 + 16 * ht + col) * PST + 32 * kt + 4 * kg;
                const uint2 lo = *reinterpret_cast<const uint2 *>(pp);
                const uint2 hi = *reinterpret_cast<const uint2 *>(pp + 16);
                pb[ht] = u32x4{lo.x, lo.y, hi.x, hi.y};
            }
            const uint16_t *tr0 = rows + (32 * kt + 4 * kg + (col >> 2)) * LS + 4 * (col & 3) + rq * DQ;
            const uint16_t *tr1 = tr0 + 16 * LS;
#pragma unroll
            for (int dt = 0; dt < DT; dt++) {
                const s16x4 lo4 = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
                    (s16x4 __attribute__((address_space(3))) *)(tr0 + 16 * dt));
                const s16x4 hi4 = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
                    (s16x4 __attribute__((address_space(3))) *)(tr1 + 16 * dt));
                const u32x4 av = {__builtin_bit_cast(uint32_t, s16x2{lo4[0], lo4[1]}),
                                  __builtin_bit_cast(uint32_t, s16x2{lo4[2], lo4[3]}),
                                  __builtin_bit_cast(uint32_t, s16x2{hi4[0], hi4[1]}),
                                  __builtin_bit_cast(uint32_t, s16x2{hi4[2], hi4[3]})};
#pragma unroll
                for (int ht = 0; ht < HT; ht++) oacc[dt][ht] = mma<CSA2_BF16>(av, pb[ht], oacc[dt][ht]);
            }
        }
    };
    for (int t = 0; t < ntl; t++) {
        const bool odd = t & 1;
        step(t, odd ? rows_b : rows_a, odd ? jsh_b : jsh_a, odd ? rows_a : rows_b, odd ? jsh_a : jsh_b);
    }

    // ---- output: out / l in bf16, staged as [head][channel] in the free row
    // buffer, written as whole rows; lse = m + ln l
    __syncthreads();
    constexpr int OS = D + 8;
    uint16_t *stage = rows_a;
#pragma unroll
    for (int ht = 0; ht < HT; ht++) {
        const int hd = hw0 + 16 * ht + col;
        const float l = l_run[ht];
        const float inv = l > 0.f ? 1.f / l : 0.f;
        uint16_t *srow = stage + hd * OS + rq * DQ + 4 * kg;
#pragma unroll
        for (int dt = 0; dt < DT; dt++) {
            const f32x4 o = oacc[dt][ht];
            const uint32_t w0 = uint32_t(f32_to_bf16_rne(o[0] * inv)) | (uint32_t(f32_to_bf16_rne(o[1] * inv)) << 16);
            const uint32_t w1 = uint32_t(f32_to_bf16_rne(o[2] * inv)) | (uint32_t(f32_to_bf16_rne(o[3] * inv)) << 16);
            *reinterpret_cast<uint2 *>(srow + 16 * dt) = make_uint2(w0, w1);
        }
        if (lse && kg == 0 && rq == 0) lse[(size_t)bq * H + hgb * HB + hd] = l > 0.f ? m_run[ht] + logf(l) : NEG_INF;
    }
    __syncthreads();
    {
        uint16_t *dst = out + ((size_t)bq * H + hgb * HB) * D;
        constexpr int OP = HB * D / 8;
#pragma unroll
        for (int i = tid; i < OP; i += NT) {
            const int r = i / (D / 8), c = i % (D / 8);
            *reinterpret_cast<u32x4 *>(dst + (size_t)r * D + 8 * c) = *reinterpret_cast<const u32x4 *>(stage + r * OS + 8 * c);
        }
    }
}

void launch_tiles(const AttnPlan &p, const void *q, const void *kv, const int32_t *idx, float scale, void *out,
                  float *lse, hipStream_t s) {
    const int nq = p.B * p.Q;
    constexpr int HB = 64;
    const int NG = p.H / HB;
    const int blocks = 8 * ((nq + 7) / 8) * NG;
    hipLaunchKernelGGL((k_attn_tiles<512, 32, 2>), dim3(blocks), dim3(512), 0, s, static_cast<const uint16_t *>(q),
                       static_cast<const uint16_t *>(kv), p.Q, p.H, p.N, idx, p.k, scale, nq,
                       static_cast<uint16_t *>(out), lse);
}

// Heads per block: as many as keep at least 256 blocks (one per compute unit),
// from 64 down to 16; the blocks that share a split's rows sit on one XCD.
template <int D, int FMT>
void launch_split(const AttnPlan &p, const void *q, const void *kv, const int32_t *idx, float scale, void *out,
                  float *lse, uint16_t *part_o, float2 *part_ml, float *part_sc, hipStream_t s,
                  const SelHandoff *sel) {
    const int npairs = p.B * p.Q * p.nsplit;
    int hb = p.H < 64 ? p.H : 64;
    while (hb > 16 && (int64_t)npairs * (p.H / hb) < 256) hb /= 2;
    const int NG = p.H / hb;
    const int blocks = 8 * ((npairs + 7) / 8) * NG;
#define CSA2_SPLIT_LAUNCH(HPW, HH)                                                                                   \
    do {                                                                                                             \
        if (sel)                                                                                                     \
            hipLaunchKernelGGL((k_attn_split<D, FMT, HPW, HH, true>), dim3(blocks), dim3(256 * HH), 0, s,             \
                               static_cast<const uint16_t *>(q), static_cast<const uint8_t *>(kv), p.Q, p.H, p.N,     \
                               idx, p.k, scale, p.nsplit, npairs, static_cast<uint16_t *>(out), lse, part_o,         \
                               part_ml, part_sc, *sel);                                                              \
        else                                                                                                         \
            hipLaunchKernelGGL((k_attn_split<D, FMT, HPW, HH, false>), dim3(blocks), dim3(256 * HH), 0, s,            \
                               static_cast<const uint16_t *>(q), static_cast<const uint8_t *>(kv), p.Q, p.H, p.N,     \
                               idx, p.k, scale, p.nsplit, npairs, static_cast<uint16_t *>(out), lse, part_o,         \
                               part_ml, part_sc, SelHandoff{});                                                      \
    } while (0)
    switch (hb) {
        case 64: CSA2_SPLIT_LAUNCH(32, 2); break;
        case 32: CSA2_SPLIT_LAUNCH(16, 2); break;
        case 16: CSA2_SPLIT_LAUNCH(16, 1); break;
        default: throw Error(CSA2_EUNSUPPORTED, "matrix-core attention needs H in {16, 32, 64, 128}");
    }
#undef CSA2_SPLIT_LAUNCH
}



}  // namespace

AttnPlan attn_plan(int q_dt, int kv_dt, int B, int Q, int H, int D, int64_t N, int k) {
    AttnPlan p{q_dt, kv_dt, B, Q, H, D, N, k, false, 1, false};
    p.mfma = q_dt == CSA2_BF16 && (kv_dt == CSA2_BF16 || kv_dt == CSA2_FP4) &&
             (H == 16 || H == 32 || H == 64 || H == 128) && (D == 64 || D == 128 || D == 256 || D == 512);
    p.nsplit = p.mfma ? (k + ATT_SPLIT - 1) / ATT_SPLIT : 1;
    // a prefill chunk (many query tokens per sequence) of bf16 rows of 512:
    // whole queries per block, no split partials
    p.tiles = p.mfma && kv_dt == CSA2_BF16 && D == 512 && H % 64 == 0 && Q >= ATT_TILES_MIN_Q && k > ATT_SPLIT;
    if (p.tiles) p.nsplit = 1;
    return p;
}

bool attn_handoff_supported(const AttnPlan &p, const SelPlan &sp) {
    // the matrix-core kernel finishes the selection in its prologue when the
    // IN bitmap is at most 1024 words (the one-block selection path)
    return p.mfma && !p.tiles && sp.certified && sp.nwords <= 1024;
}

bool attn_supported(const AttnPlan &p) {
    if (p.mfma) return (int64_t)p.B * p.Q * p.nsplit * (p.H / 16) + 8 * (p.H / 16) <= INT32_MAX;  // blocks fit an int
    return (p.D + p.k) <= 16384;
}

size_t attn_workspace(const AttnPlan &p) {
    if (!p.mfma || p.tiles || p.nsplit == 1) return 0;
    Carve c(nullptr, 0);
    c.take<uint16_t>((size_t)p.B * p.Q * p.nsplit * p.H * p.D);
    c.take<float2>((size_t)p.B * p.Q * p.nsplit * p.H);
    c.take<float>((size_t)p.B * p.Q * p.nsplit * p.H * 4);
    return c.used;
}


void attn_run(const AttnPlan &p, const void *q, const void *kv, const int32_t *idx, float scale, void *out,
              float *lse, void *ws, size_t ws_bytes, hipStream_t s, const SelHandoff *sel) {
    const int BQ = p.B * p.Q;
    if (!p.mfma) {
        size_t lds = sizeof(float) * ((size_t)p.D + p.k);
        hipLaunchKernelGGL(k_attn_valu, dim3(p.H, BQ), dim3(256), lds, s, q, p.q_dt,
                           static_cast<const uint8_t *>(kv), p.kv_dt, p.Q, p.H, p.D, p.N, idx, p.k, scale, out, lse);
        check_launch("attention (vector)");
        return;
    }
    if (p.tiles) {
        if (sel) throw Error(CSA2_EINTERNAL, "the prefill attention takes finished indices");
        launch_tiles(p, q, kv, idx, scale, out, lse, s);
        check_launch("attention (prefill tiles)");
        return;
    }
    uint16_t *part_o = nullptr;
    float2 *part_ml = nullptr;
    float *part_sc = nullptr;
    if (p.nsplit > 1) {
        Carve c(ws, ws_bytes);
        part_o = c.take<uint16_t>((size_t)BQ * p.nsplit * p.H * p.D);
        part_ml = c.take<float2>((size_t)BQ * p.nsplit * p.H);
        part_sc = c.take<float>((size_t)BQ * p.nsplit * p.H * 4);
        if (c.used > ws_bytes) throw Error(CSA2_EWORKSPACE, "attention workspace too small");
    }
#define CSA2_ATT_CASE(d)                                                                             \
    case d:                                                                                          \
        if (p.kv_dt == CSA2_FP4) launch_split<d, CSA2_FP4>(p, q, kv, idx, scale, out, lse, part_o, part_ml, part_sc, s, sel); \
        else launch_split<d, CSA2_BF16>(p, q, kv, idx, scale, out, lse, part_o, part_ml, part_sc, s, sel);                   \
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
        const int64_t threads = (int64_t)BQ * p.H * (p.D / COMB_CPT);
        hipLaunchKernelGGL(k_attn_combine, dim3((unsigned)((threads + 255) / 256)), dim3(256), 0, s, part_o, part_ml, part_sc,
                           BQ, p.H, p.D, p.nsplit, out, p.q_dt, lse);
        check_launch("attention combine");
    }
}

}  // namespace csa2
