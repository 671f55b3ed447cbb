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
// Matrix-core kernel: a block serves all heads of one query over a fixed split
// of 128 selected entries (the split depends only on k, so a query's result
// does not depend on the batch), one wave per 16 heads.  The gathered rows are
// staged once per block in LDS as bf16 (FP4 rows decoded on the way in, to
// fp16, where they are also exact), S^T = C Q^T runs on the 16x16x32
// matrix-core instruction of that type with the rows as the A operand, the
// online softmax keeps one running max per head, and O^T = C^T P^T reuses the
// same LDS rows (read transposed) with P^T taken straight from the S^T result
// registers.  Splits are merged by a small combine kernel.
#include "internal.h"

namespace csa2 {

constexpr int ATT_SUB = 32;  // entries per tile

// Selected entries per split: fixed, so that a query's result does not depend
// on the batch it is computed in.  (Longer splits halve the combine traffic but
// leave each block a longer chain of gathers; measured slower at k = 2048.)
constexpr int ATT_SPLIT = 128;

namespace {

constexpr float NEG_INF = -__builtin_inff();

// 4-bit E2M1 code -> binary32 bits (OCP MX element: bias 1, code 0bS001 = 0.5).
__device__ __forceinline__ uint32_t e2m1_bits(uint32_t c) {
    const uint32_t e = (c >> 1) & 3u, mb = c & 1u;
    const uint32_t mag = e ? (((e + 126u) << 23) | (mb << 22)) : (mb ? 0x3f000000u : 0u);
    return mag | ((c & 8u) << 28);
}
// FP4 row scale byte -> float: its E4M3 ("FN") value (bias 7; exponent field
// 0 is m * 2^-9), except the NaN code S.1111.111, which saturates to +-448.
__device__ __forceinline__ float e4m3_val(uint32_t s) {
    const uint32_t e = (s >> 3) & 15u, mt = s & 7u;
    float mag = e ? __uint_as_float(((e + 120u) << 23) | (mt << 20)) : (float)mt * 0.001953125f;
    if ((s & 0x7fu) == 0x7fu) mag = 448.f;
    return (s & 0x80u) ? -mag : mag;
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
// Block = one query x one split of the selected entries x HB groups of 16
// heads; wave w serves heads 16 (HB g + w % HB) .. +15 and, with DS = 2, half of the output channels (the
// two waves of a head group both compute that group's logits).  Per 32-entry tile: all threads gather the rows into an
// LDS buffer (bf16 rows as is, FP4 rows decoded to fp16), the next tile's rows
// are already in flight in registers; each wave computes S^T = C Q^T (rows as
// the A operand), the online softmax of its 16 heads, and O^T += C^T P^T with
// the C^T operand read by the LDS transpose load: lane r of each 16-lane group
// points at 4 consecutive channels of one row, and lane i receives channel i
// of 4 consecutive rows.

typedef short __attribute__((ext_vector_type(4))) s16x4;
typedef float __attribute__((ext_vector_type(2))) f32x2;
typedef __bf16 __attribute__((ext_vector_type(2))) bf16x2v;  // converted to with round-to-nearest-even
typedef _Float16 __attribute__((ext_vector_type(2))) f16x2;

// FP4 chunk (32 channels: 16 code bytes) with the two E4M3 scales of its
// 16-channel halves -> 32 fp16 values.  The conversion instruction applies the
// scale's power of two; the scale's mantissa (1 + m/8, at most 3 bits) is
// applied by an fp16 multiply.  Every product has <= 5 significant bits and a
// magnitude in [2^-10, 3072], so both steps are exact.
__device__ __forceinline__ void fp4_chunk_to_f16(u32x4 codes, uint32_t sc2, uint32_t *dst16) {
#pragma unroll
    for (int half = 0; half < 2; half++) {
        const float s = e4m3_val((sc2 >> (8 * half)) & 0xffu);
        const uint32_t sb = __float_as_uint(s);
        float pow2 = __uint_as_float(sb & 0x7f800000u);
        uint32_t fbits = 0x3c00u | ((sb >> 13) & 0x3ffu) | ((sb >> 16) & 0x8000u);
        if (s == 0.f) {
            pow2 = 1.f;
            fbits = 0u;
        }
        const f16x2 f = __builtin_bit_cast(f16x2, fbits | (fbits << 16));
#pragma unroll
        for (int wi = 0; wi < 2; wi++) {
            const uint32_t word = codes[half * 2 + wi];
            f16x2 v0 = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(word, pow2, 0) * f;
            f16x2 v1 = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(word, pow2, 1) * f;
            f16x2 v2 = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(word, pow2, 2) * f;
            f16x2 v3 = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(word, pow2, 3) * f;
            uint32_t *o = dst16 + (half * 2 + wi) * 4;
            o[0] = __builtin_bit_cast(uint32_t, v0);
            o[1] = __builtin_bit_cast(uint32_t, v1);
            o[2] = __builtin_bit_cast(uint32_t, v2);
            o[3] = __builtin_bit_cast(uint32_t, v3);
        }
    }
}

template <int D, int FMT>
struct TileGather {
    // bf16: a row is D/8 16-byte chunks; FP4: a row is D/32 chunks of 16 code
    // bytes (32 channels) plus 2 scale bytes each.
    static constexpr int CPR = FMT == CSA2_FP4 ? D / 32 : D / 8;
    static constexpr int CHUNKS = ATT_SUB * CPR;
    static constexpr int ROWB = FMT == CSA2_FP4 ? D / 2 + D / 16 : 2 * D;
};

// Loads of one tile's rows into registers: every lane loads (entries of -1
// read row 0 and are flagged in bit 31 of sbuf, then zeroed by gather_store),
// so that no branch or copy stands between the loads and they all fly at once.
template <int D, int FMT, int NT>
__device__ __forceinline__ void gather_issue(const uint8_t *kvb, const int32_t *jt, u32x4 *buf, uint32_t *sbuf) {
    using G = TileGather<D, FMT>;
    constexpr int PER = (G::CHUNKS + NT - 1) / NT;
#pragma unroll
    for (int u = 0; u < PER; u++) {
        const int c = threadIdx.x + u * NT;
        const int cs = c < G::CHUNKS ? c : 0;
        const int r = cs / G::CPR, cc = cs % G::CPR;
        const int j = jt[r];
        const uint8_t *row = kvb + (size_t)(j >= 0 ? j : 0) * G::ROWB;
        buf[u] = *reinterpret_cast<const u32x4 *>(row + cc * 16);
        uint32_t sc = 0;
        if constexpr (FMT == CSA2_FP4) sc = *reinterpret_cast<const uint16_t *>(row + D / 2 + cc * 2);
        sbuf[u] = sc | (j < 0 ? 0x80000000u : 0u);
    }
}

template <int D, int FMT, int NT>
__device__ __forceinline__ void gather_store(uint16_t *T, const u32x4 *buf, const uint32_t *sbuf) {
    using G = TileGather<D, FMT>;
    constexpr int PER = (G::CHUNKS + NT - 1) / NT;
    constexpr int LS = D + 8;
#pragma unroll
    for (int u = 0; u < PER; u++) {
        const int c = threadIdx.x + u * NT;
        if (c >= G::CHUNKS) continue;
        const int r = c / G::CPR, cc = c % G::CPR;
        const bool skip = sbuf[u] >> 31;  // no entry: the row is zero
        if constexpr (FMT == CSA2_FP4) {
            uint32_t o[16];
            fp4_chunk_to_f16(skip ? u32x4{0u, 0u, 0u, 0u} : buf[u], skip ? 0u : sbuf[u] & 0xffffu, o);
            uint32_t *dst = reinterpret_cast<uint32_t *>(T + r * LS + cc * 32);
#pragma unroll
            for (int q4 = 0; q4 < 4; q4++)
                reinterpret_cast<u32x4 *>(dst)[q4] = u32x4{o[4 * q4], o[4 * q4 + 1], o[4 * q4 + 2], o[4 * q4 + 3]};
        } else {
            *reinterpret_cast<u32x4 *>(T + r * LS + cc * 8) = skip ? u32x4{0u, 0u, 0u, 0u} : buf[u];
        }
    }
}

// ------------------------------------------------ selection finish (fused)
// A block's share of the certified top-k, finished from the selection's
// records in three steps.  The attention itself only needs the selected SET;
// its blocks take the entries in this order: the IN entries in slot order
// (positions 0 .. |IN|-1), then the best K - |IN| band entries in rank order
// (binary64 score descending, slot ascending).  A split's first tile usually
// holds IN entries only, so its rows are in flight while the band is ranked.
// The index output is the selected set in slot order, written after the
// ranking.  Redundant across the query's blocks, but short, and it saves a
// dependent launch.  `scratch` (bytes available: cap) holds the bitmap and
// the band until sel_split_idx returns.
struct BandEntA {
    uint64_t key;
    int32_t slot;
    uint32_t nslot;  // ~slot: ascending slot order as descending unsigned order
};

struct SplitSel {
    int32_t in_cnt, nb;  // |IN| and the band size
    bool in_lds;         // the band is staged in LDS
};

__device__ __forceinline__ int32_t sel_entry(const SelHandoff &sel, int bq, int32_t slot) {
    return sel.cand ? sel.cand[(size_t)bq * sel.n + slot] : slot;
}

// Popcount scan of the bitmap: thread tid owns words [tid * per, ...); returns
// its first position and the block total.
template <int NT>
__device__ __forceinline__ uint32_t bitmap_scan(const uint32_t *bm, int64_t nwords, uint32_t *red, uint32_t &mine,
                                                uint32_t &tot) {
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int64_t per = (nwords + NT - 1) / NT;
    const int64_t w0 = (int64_t)tid * per;
    mine = 0;
    for (int64_t w = w0; w < w0 + per && w < nwords; w++) mine += __builtin_popcount(bm[w]);
    const uint32_t incl = wave_incl_scan_u32(mine);
    if (lane == 63) red[wave] = incl;
    __syncthreads();
    uint32_t before = 0;
    tot = 0;
#pragma unroll
    for (int i = 0; i < NT / 64; i++) {
        const uint32_t x = red[i];
        before += i < wave ? x : 0u;
        tot += x;
    }
    return before + incl - mine;
}

// Step 1: the records into LDS (IN bitmap, band entries with their keys) and
// the split's IN positions into jsh (-1 elsewhere).  Ends with jsh's IN part
// visible to the block.
template <int NT, int SPLIT>
__device__ SplitSel sel_split_in(const SelHandoff &sel, int bq, int e_begin, int ne, uint32_t *scratch, size_t cap,
                                 int32_t *jsh, uint32_t *red) {
    const int tid = threadIdx.x;
    const int64_t nwords = sel.nwords;
    const int64_t nw4 = (nwords + 3) & ~int64_t(3);
    uint32_t *bm = scratch;
    BandEntA *ent = reinterpret_cast<BandEntA *>(scratch + nw4);
    const uint32_t *gbm = sel.bitmap + (size_t)bq * nwords;
    const int32_t *list = sel.band + (size_t)bq * sel.band_cap;
    const double *bs = sel.band_score + (size_t)bq * sel.band_cap;
    // One round of loads before anything waits: the first NT band entries
    // (speculatively, before the count is known; past the capacity they read
    // the last one), the bitmap (four words per load where the rows are
    // 16-byte aligned) and the target record, which is used only after them.
    const int32_t spec_i = tid < sel.band_cap ? tid : (int32_t)sel.band_cap - 1;
    const int32_t sl0 = list[spec_i];
    const double sc0 = bs[spec_i];
    constexpr int U = 4;  // NT * U * 4 words per round
    const bool vec = (nwords & 3) == 0;
    const int64_t nq = nwords >> 2;
    u32x4 v[U];
    if (vec) {
#pragma unroll
        for (int u = 0; u < U; u++) {
            const int64_t qi = tid + (int64_t)NT * u;
            v[u] = reinterpret_cast<const u32x4 *>(gbm)[qi < nq ? qi : nq - 1];
        }
    }
    const SelTarget t = sel.sq[bq].t[0];
    SplitSel st;
    st.in_cnt = t.in_cnt;
    st.nb = t.band_cnt;
    st.in_lds = st.nb <= (int32_t)((cap - (size_t)nw4 * 4) / sizeof(BandEntA));
    if (vec) {
#pragma unroll
        for (int u = 0; u < U; u++) {
            const int64_t qi = tid + (int64_t)NT * u;
            if (qi < nq) reinterpret_cast<u32x4 *>(bm)[qi] = v[u];
        }
        for (int64_t q0 = (int64_t)NT * U; q0 < nq; q0 += (int64_t)NT * U) {
#pragma unroll
            for (int u = 0; u < U; u++) {
                const int64_t qi = q0 + tid + (int64_t)NT * u;
                v[u] = reinterpret_cast<const u32x4 *>(gbm)[qi < nq ? qi : nq - 1];
            }
#pragma unroll
            for (int u = 0; u < U; u++) {
                const int64_t qi = q0 + tid + (int64_t)NT * u;
                if (qi < nq) reinterpret_cast<u32x4 *>(bm)[qi] = v[u];
            }
        }
    } else {
        for (int64_t w = tid; w < nwords; w += NT) bm[w] = gbm[w];
    }
    for (int e = tid; e < SPLIT; e += NT) jsh[e] = -1;
    if (st.in_lds) {
        if (tid < st.nb) {
            BandEntA e;
            e.key = dkey(sc0);
            e.slot = sl0;
            e.nslot = ~(uint32_t)e.slot;
            ent[tid] = e;
        }
        for (int32_t i = tid + NT; i < st.nb; i += NT) {
            BandEntA e;
            e.key = dkey(bs[i]);
            e.slot = list[i];
            e.nslot = ~(uint32_t)e.slot;
            ent[i] = e;
        }
    }
    __syncthreads();
    uint32_t mine, tot;
    uint32_t pos = bitmap_scan<NT>(bm, nwords, red, mine, tot);
    const uint32_t lo = (uint32_t)e_begin, hi = (uint32_t)(e_begin + ne);
    if (pos < hi && pos + mine > lo) {
        const int64_t per = (nwords + NT - 1) / NT;
        const int64_t w0 = (int64_t)tid * per;
        for (int64_t w = w0; w < w0 + per && w < nwords; w++) {
            uint32_t bits = bm[w];
            while (bits) {
                const int b = __builtin_ctz(bits);
                bits &= bits - 1;
                if (pos >= lo && pos < hi) jsh[pos - lo] = sel_entry(sel, bq, (int32_t)(w * 32 + b));
                pos++;
            }
        }
    }
    __syncthreads();
    return st;
}

// Step 2: rank the band; the best r = K - |IN| entries join the bitmap, and
// those whose positions |IN| + rank fall in the split go into jsh.  issue()
// is called once (it starts the first tile's row loads when they are known):
// on the common path right after the ranking's LDS reads, so that the loads
// fly during the ranking.  Ends with jsh complete.
template <int NT, int SPLIT, class Issue>
__device__ void sel_split_band(const SelHandoff &sel, int bq, int K, const SplitSel &st, int e_begin, int ne,
                               uint32_t *scratch, size_t cap, int32_t *jsh, Issue &&issue) {
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int64_t nw4 = (sel.nwords + 3) & ~int64_t(3);
    uint32_t *bm = scratch;
    const u32x4 *ent4 = reinterpret_cast<const u32x4 *>(scratch + nw4);
    const int32_t nb = st.nb, r = K - st.in_cnt;
    const int32_t *list = sel.band + (size_t)bq * sel.band_cap;
    const double *bs = sel.band_score + (size_t)bq * sel.band_cap;
    // entry with slot si and rank rk (< r) is selected
    auto take = [&](int32_t si, int32_t rk) {
        atomicOr(&bm[si >> 5], 1u << (si & 31));
        const int32_t p = st.in_cnt + rk - e_begin;
        if (p >= 0 && p < ne) jsh[p] = sel_entry(sel, bq, si);
    };
    if (r > 0 && nb > 0 && st.in_lds && nb <= NT &&
        (size_t)(nw4 + 4 * nb) * 4 + (size_t)(NT / 64) * NT * 4 <= cap) {
        // Lane l of chunk c holds entry i = 64 c + l; wave w takes its share of
        // the partners j, read from LDS as broadcasts.  j is ahead of i iff
        // (key_j, ~slot_j) > (key_i, ~slot_i) as 96-bit unsigned numbers, i.e.
        // iff the subtraction (key_i, ~slot_i) - (key_j, ~slot_j) borrows: three
        // chained subtractions and an add of the borrow, all on the vector
        // unit.  The waves' counts meet in LDS and thread i sums them.
        constexpr int NW = NT / 64;
        constexpr int MAXC = NT / 64;
        uint32_t *rkp = scratch + nw4 + 4 * nb;
        const int nch = (nb + 63) / 64;
        u32x4 ic[MAXC];
#pragma unroll
        for (int c = 0; c < MAXC; c++) {
            const int i = 64 * c + lane;
            ic[c] = c < nch ? ent4[i < nb ? i : 0] : u32x4{0u, 0u, 0u, 0u};
        }
        const bool act = tid < nb;
        const u32x4 me = ent4[act ? tid : 0];
        const int32_t my_e = sel_entry(sel, bq, (int32_t)me[2]);  // before the row loads
        issue();  // global loads go out after these LDS reads
        uint32_t rk[MAXC];
#pragma unroll
        for (int c = 0; c < MAXC; c++) rk[c] = 0;
        const int jper = (nb + NW - 1) / NW;
        const int j0 = __builtin_amdgcn_readfirstlane(wave * jper);
        const int j1 = __builtin_amdgcn_readfirstlane(min(nb, j0 + jper));
        // (key lo, key hi, slot, ~slot) of partner j against every chunk
        auto count = [&](const u32x4 &o) {
#pragma unroll
            for (int c = 0; c < MAXC; c++) {
                if (c < nch) {
                    uint32_t d;
                    asm volatile(
                        "v_sub_co_u32 %0, vcc, %2, %3\n\t"
                        "v_subb_co_u32 %0, vcc, %4, %5, vcc\n\t"
                        "v_subb_co_u32 %0, vcc, %6, %7, vcc\n\t"
                        "v_addc_co_u32 %1, vcc, 0, %1, vcc"
                        : "=&v"(d), "+v"(rk[c])
                        : "v"(ic[c][3]), "v"(o[3]), "v"(ic[c][0]), "v"(o[0]), "v"(ic[c][1]), "v"(o[1])
                        : "vcc");
                }
            }
        };
        int j = j0;
        for (; j + 4 <= j1; j += 4) {
            u32x4 o[4];
#pragma unroll
            for (int u = 0; u < 4; u++) o[u] = ent4[j + u];
#pragma unroll
            for (int u = 0; u < 4; u++) count(o[u]);
        }
        for (; j < j1; j++) count(ent4[j]);
#pragma unroll
        for (int c = 0; c < MAXC; c++)
            if (c < nch) rkp[wave * NT + 64 * c + lane] = rk[c];
        __syncthreads();
        if (act) {
            uint32_t rank = 0;
#pragma unroll
            for (int w = 0; w < NW; w++) rank += rkp[w * NT + tid];
            if (rank < (uint32_t)r) {
                const int32_t si = (int32_t)me[2];
                atomicOr(&bm[si >> 5], 1u << (si & 31));
                const int32_t p = st.in_cnt + (int32_t)rank - e_begin;
                if (p >= 0 && p < ne) jsh[p] = my_e;
            }
        }
    } else if (r > 0 && nb > 0) {
        // entry i is ranked by P consecutive lanes, each comparing a 1/P share
        const int P = nb * 8 <= NT ? 8 : nb * 4 <= NT ? 4 : nb * 2 <= NT ? 2 : 1;
        const int per = NT / P;
        for (int32_t i0 = 0; i0 < nb; i0 += per) {
            const int32_t i = i0 + tid / P;
            const int ep = tid % P;
            const bool act = i < nb;
            const int32_t ii = act ? i : 0;
            int32_t rank = 0;
            uint64_t ki;
            int32_t si;
            if (st.in_lds) {
                const u32x4 me = ent4[ii];
                ki = (uint64_t)me[0] | ((uint64_t)me[1] << 32);
                si = (int32_t)me[2];
                for (int32_t j0 = ep; j0 < nb; j0 += 8 * P) {
                    u32x4 bj[8];
#pragma unroll
                    for (int u = 0; u < 8; u++) {
                        const int32_t j = j0 + u * P;
                        bj[u] = ent4[j < nb ? j : ii];  // past the end: compare with itself (counts 0)
                    }
#pragma unroll
                    for (int u = 0; u < 8; u++) {
                        const uint64_t kj = (uint64_t)bj[u][0] | ((uint64_t)bj[u][1] << 32);
                        rank += (int)((kj > ki) | ((kj == ki) & ((int32_t)bj[u][2] < si)));
                    }
                }
            } else {
                ki = dkey(bs[ii]);
                si = list[ii];
                for (int32_t j = ep; j < nb; j += P) {
                    const uint64_t kj = dkey(bs[j]);
                    const int32_t sj = list[j];
                    rank += (int)((kj > ki) | ((kj == ki) & (sj < si)));
                }
            }
            if (P >= 2) rank = bfly1(rank, OpAdd{});
            if (P >= 4) rank = bfly2(rank, OpAdd{});
            if (P >= 8) rank = bfly4(rank, OpAdd{});
            if (act && ep == 0 && rank < r) take(si, rank);
        }
        __builtin_amdgcn_s_waitcnt(0);  // this path's own loads are done before the rows go out
        issue();
    } else {
        issue();
    }
    __syncthreads();
}

// Step 3: the index output, the selected set in slot order (its split's share,
// -1 past the count), and the count (split 0).  Ends with the scratch free.
template <int NT>
__device__ void sel_split_idx(const SelHandoff &sel, int bq, int K, int e_begin, int ne, bool first,
                              const uint32_t *scratch, uint32_t *red) {
    const int tid = threadIdx.x;
    const int64_t nwords = sel.nwords;
    const uint32_t *bm = scratch;
    uint32_t mine, tot;
    uint32_t pos = bitmap_scan<NT>(bm, nwords, red, mine, tot);
    const int32_t kept = (int32_t)(tot < (uint32_t)K ? tot : (uint32_t)K);
    const uint32_t lo = (uint32_t)e_begin, hi = (uint32_t)(e_begin + ne);
    int32_t *orow = sel.idx + (size_t)bq * K + e_begin;
    // one loop per mapping, so that the identity mapping waits for no load
    auto scatter = [&](auto map) {
        const int64_t per = (nwords + NT - 1) / NT;
        const int64_t w0 = (int64_t)tid * per;
        for (int64_t w = w0; w < w0 + per && w < nwords; w++) {
            uint32_t bits = bm[w];
            while (bits) {
                const int b = __builtin_ctz(bits);
                bits &= bits - 1;
                if (pos >= lo && pos < hi) orow[pos - lo] = map((int32_t)(w * 32 + b));
                pos++;
            }
        }
    };
    if (pos < hi && pos + mine > lo) {
        if (sel.cand) {
            const int32_t *cq = sel.cand + (size_t)bq * sel.n;
            scatter([&](int32_t sl) { return cq[sl]; });
        } else {
            scatter([](int32_t sl) { return sl; });
        }
    }
    for (int e = (kept > e_begin ? kept - e_begin : 0) + tid; e < ne; e += NT) orow[e] = -1;
    if (first && tid == 0 && sel.count) sel.count[bq] = kept;
    __syncthreads();
}

// Balanced pairwise sum of 1, 2 or 4 partial tiles.
template <int NPS>
__device__ __forceinline__ f32x4 tree_sum(const f32x4 *p) {
    if constexpr (NPS == 1) return p[0];
    else if constexpr (NPS == 2) return p[0] + p[1];
    else return (p[0] + p[1]) + (p[2] + p[3]);
}


// Block order: the NG blocks that share one (query, split) -- one per group
// of HB x 16 heads -- get linear ids congruent mod 8, so that the round-robin
// dispatch puts them on one XCD and they gather the split's rows through one
// L2.  Ids past the last (query, split) pair exit at once.
template <int D, int FMT, int HB, int DS, int SPLIT, bool FROMSEL>
__global__ __launch_bounds__(64 * HB * DS, 1) void k_attn_mfma(const uint16_t *__restrict__ q, const uint8_t *__restrict__ kv,
                                                          int Q, int H, int64_t N, const int32_t *__restrict__ idx,
                                                          int k, float scale, int nsplit, int npairs,
                                                          uint16_t *__restrict__ out, float *__restrict__ lse,
                                                          uint16_t *__restrict__ part_o, float2 *__restrict__ part_ml,
                                                          float *__restrict__ part_sc, SelHandoff sel) {
    constexpr int NT = 64 * HB * DS;
    constexpr int KS = D / 32 / DS;  // contraction steps of S owned by this wave (its channel part)
    constexpr int SP = D >= 256 ? 4 : 2;  // channel parts of the S contraction, for every DS
    static_assert(SP % DS == 0 && (D / 32) % SP == 0, "S parts must split evenly over the waves");
    constexpr int LP = SP / DS;       // parts contracted by this wave
    constexpr int PS = KS / LP;       // steps per part
    constexpr int DT = D / 16 / DS;  // 16-wide d tiles of O owned by this wave
    constexpr int LS = D + 8;   // LDS row stride in 16-bit elements (16-byte pad)
    using G = TileGather<D, FMT>;
    constexpr int PER = (G::CHUNKS + NT - 1) / NT;
    __shared__ __attribute__((aligned(16))) uint16_t tile[2][ATT_SUB * LS];
    __shared__ __attribute__((aligned(16))) int32_t jsh[SPLIT];
    // partial logits of each wave's channel part, summed over the head group's DS waves
    __shared__ __attribute__((aligned(16))) f32x4 spart[DS > 1 ? 64 * HB * DS * 2 : 1];

    const int NG = H / (16 * HB);
    const int L = blockIdx.x;
    const int pair = (L / (8 * NG)) * 8 + (L % 8);
    const int hgb = (L % (8 * NG)) / 8;
    if (pair >= npairs) return;
    const int split = pair % nsplit;
    const int bq = pair / nsplit;
    const int b = bq / Q;
    const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
    const int col = lane & 15, kg = lane >> 4;
    const int hg = hgb * HB + wave % HB;  // this wave's 16 heads
    const int dpart = wave / HB;          // this wave's channel part: S over it, O for it
    const int dt0 = dpart * DT;           // first d tile of this wave

    const int e_begin = split * SPLIT;
    const int e_end = min(k, e_begin + SPLIT);
    const int ne = e_end - e_begin;
    const uint8_t *kvb = kv + (size_t)b * N * G::ROWB;
    // Query heads as the B operand of S^T = C Q^T (fp16 for FP4 rows), in flight from the start.
    u32x4 qf[KS];
    const uint16_t *qrow = q + ((size_t)bq * H + hg * 16 + col) * D + 8 * kg + 32 * KS * dpart;
#pragma unroll
    for (int s = 0; s < KS; s++) qf[s] = *reinterpret_cast<const u32x4 *>(qrow + 32 * s);

    const int ntiles = (ne + ATT_SUB - 1) / ATT_SUB;
    u32x4 buf[PER];
    uint32_t sbuf[PER];
    if constexpr (FROMSEL) {
        // the selected set from the certified selection's records (LDS scratch in the tile buffers)
        __shared__ uint32_t sred[NT / 64];
        uint32_t *scr = reinterpret_cast<uint32_t *>(tile[0]);
        const SplitSel st = sel_split_in<NT, SPLIT>(sel, bq, e_begin, ne, scr, sizeof(tile), jsh, sred);
        // the first tile's rows go out now if its entries are all IN entries
        const bool early = e_begin + min(ATT_SUB, ne) <= st.in_cnt;
        // (issued unconditionally: a branch around the loads would make later
        // waits for other loads wait for these too; reissued below if not early)
        sel_split_band<NT, SPLIT>(sel, bq, k, st, e_begin, ne, scr, sizeof(tile), jsh,
                                  [&]() { gather_issue<D, FMT, NT>(kvb, jsh, buf, sbuf); });
        sel_split_idx<NT>(sel, bq, k, e_begin, ne, split == 0, scr, sred);
        if (!early) gather_issue<D, FMT, NT>(kvb, jsh, buf, sbuf);
    } else {
        const int32_t *irow = idx + (size_t)bq * k + e_begin;
        for (int e = threadIdx.x; e < SPLIT; e += NT) {
            int j = e < ne ? irow[e] : -1;
            jsh[e] = (j >= 0 && j < N) ? j : -1;  // out-of-range entries are skipped like -1
        }
        __syncthreads();  // jsh ready
        if (ntiles > 0) gather_issue<D, FMT, NT>(kvb, jsh, buf, sbuf);
    }
    float qscale = scale;
    if constexpr (FMT == CSA2_FP4) {
        // the power-of-two scale covers the whole rows of the 16 heads, so that the
        // DS waves sharing them contract with the same scaled q
        float amax = 0.f;
        const uint16_t *qall = qrow - 32 * KS * dpart;
#pragma unroll
        for (int s = 0; s < KS * DS; s++) {
            const u32x4 v = *reinterpret_cast<const u32x4 *>(qall + 32 * s);
#pragma unroll
            for (int e = 0; e < 4; e++)
                amax = fmaxf(amax, fmaxf(fabsf(bf16_to_f32(v[e] & 0xffffu)), fabsf(bf16_to_f32(v[e] >> 16))));
        }
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

    if (ntiles > 0) gather_store<D, FMT, NT>(tile[0], buf, sbuf);
    __syncthreads();
    for (int t = 0; t < ntiles; t++) {
        if (t + 1 < ntiles) gather_issue<D, FMT, NT>(kvb, jsh + (t + 1) * ATT_SUB, buf, sbuf);
        const uint16_t *T = tile[t & 1];
        const int32_t *jt = jsh + t * ATT_SUB;
        // ---- S^T[e][h] for the two 16-entry halves. The contraction is cut into SP
        // channel parts summed as a balanced tree, the same for every DS: this wave
        // contracts its SP/DS parts and adds them, the DS waves' sums are then added.
        f32x4 st[2];
#pragma unroll
        for (int h2 = 0; h2 < 2; h2++) {
            const uint16_t *arow = T + (h2 * 16 + col) * LS + 8 * kg + 32 * KS * dpart;
            f32x4 pp[LP];
#pragma unroll
            for (int lp = 0; lp < LP; lp++) {
                pp[lp] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
                for (int s = 0; s < PS; s++) {
                    const u32x4 av = *reinterpret_cast<const u32x4 *>(arow + 32 * (lp * PS + s));
                    pp[lp] = mma<FMT>(av, qf[lp * PS + s], pp[lp]);
                }
            }
            st[h2] = tree_sum<LP>(pp);
        }
        if constexpr (DS > 1) {
#pragma unroll
            for (int h2 = 0; h2 < 2; h2++) spart[(wave * 64 + lane) * 2 + h2] = st[h2];
            __syncthreads();
#pragma unroll
            for (int h2 = 0; h2 < 2; h2++) {
                f32x4 pp[DS];
#pragma unroll
                for (int p2 = 0; p2 < DS; p2++) pp[p2] = spart[(((wave % HB) + p2 * HB) * 64 + lane) * 2 + h2];
                st[h2] = tree_sum<DS>(pp);
            }
        }
        // ---- online softmax for head col; this lane holds entries 16 h2 + 4 kg + i
        float a[8];
        float mt = NEG_INF;
        // this lane's 8 entries (16 h2 + 4 kg + i): -1 marks an empty one
        const int4 jv[2] = {*reinterpret_cast<const int4 *>(jt + 4 * kg), *reinterpret_cast<const int4 *>(jt + 16 + 4 * kg)};
#pragma unroll
        for (int h2 = 0; h2 < 2; h2++)
#pragma unroll
            for (int i = 0; i < 4; i++) {
                const int jj = i == 0 ? jv[h2].x : i == 1 ? jv[h2].y : i == 2 ? jv[h2].z : jv[h2].w;
                const float v = jj >= 0 ? st[h2][i] * qscale : NEG_INF;
                a[h2 * 4 + i] = v;
                mt = fmaxf(mt, v);
            }
        mt = bfly32(bfly16(mt, OpMax{}), OpMax{});
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
            else pk[x / 2] = __builtin_bit_cast(uint32_t, __builtin_convertvector((f32x2{p0, p1}), bf16x2v));
        }
        l_run = l_run * alpha + psum;
        m_run = m_new;
        const u32x4 pb = {pk[0], pk[1], pk[2], pk[3]};
        // ---- O^T[d][h] += C^T[d][e] P^T[e][h]: A operand element x is row
        // 16 (x/4) + 4 kg + x%4, channel 16 dt + col (two transpose loads).
        const uint16_t *tr0 = T + (4 * kg + (col >> 2)) * LS + 4 * (col & 3);
        const uint16_t *tr1 = tr0 + 16 * LS;
#pragma unroll
        for (int dt = 0; dt < DT; dt++) {
            const s16x4 lo4 = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
                (s16x4 __attribute__((address_space(3))) *)(tr0 + 16 * (dt0 + dt)));
            const s16x4 hi4 = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
                (s16x4 __attribute__((address_space(3))) *)(tr1 + 16 * (dt0 + dt)));
            const u32x4 av = {__builtin_bit_cast(uint32_t, s16x2{lo4[0], lo4[1]}),
                              __builtin_bit_cast(uint32_t, s16x2{lo4[2], lo4[3]}),
                              __builtin_bit_cast(uint32_t, s16x2{hi4[0], hi4[1]}),
                              __builtin_bit_cast(uint32_t, s16x2{hi4[2], hi4[3]})};
            o[dt] = o[dt] * alpha;
            o[dt] = mma<FMT>(av, pb, o[dt]);
        }
        if (t + 1 < ntiles) gather_store<D, FMT, NT>(tile[(t + 1) & 1], buf, sbuf);
        __syncthreads();
    }

    // ---- write this wave's 16 heads: lane holds O^T[16 dt + 4 kg + r][col]
    l_run = bfly32(bfly16(l_run, OpAdd{}), OpAdd{});
    const int h = hg * 16 + col;
    if (nsplit == 1) {
        const float inv = l_run > 0.f ? 1.f / l_run : 0.f;
        uint16_t *orow = out + ((size_t)bq * H + h) * D + 16 * dt0 + 4 * kg;
#pragma unroll
        for (int dt = 0; dt < DT; dt++) {
            const uint32_t w0 = uint32_t(f32_to_bf16_rne(o[dt][0] * inv)) | (uint32_t(f32_to_bf16_rne(o[dt][1] * inv)) << 16);
            const uint32_t w1 = uint32_t(f32_to_bf16_rne(o[dt][2] * inv)) | (uint32_t(f32_to_bf16_rne(o[dt][3] * inv)) << 16);
            *reinterpret_cast<uint2 *>(orow + 16 * dt) = make_uint2(w0, w1);
        }
        if (lse && kg == 0 && dt0 == 0) lse[(size_t)bq * H + h] = l_run > 0.f ? m_run + logf(l_run) : NEG_INF;
    } else {
        const size_t pi = ((size_t)bq * H + h) * nsplit + split;  // a head's splits are adjacent
        // the partial row in fp16 under a power-of-two scale per quarter of the
        // channels (this wave's part spans 4 / DS quarters): its largest
        // magnitude lands in [2^14, 2^15), so every value keeps fp16's 11
        // significant bits and none overflows
        float mx = 0.f;
#pragma unroll
        for (int dt = 0; dt < DT; dt++)
#pragma unroll
            for (int r = 0; r < 4; r++) mx = fmaxf(mx, fabsf(o[dt][r]));
        mx = bfly32(bfly16(mx, OpMax{}), OpMax{});
        int ex = 0;
        if (mx > 0.f && mx <= __FLT_MAX__) {
            frexpf(mx, &ex);
            ex = min(max(ex - 15, -120), 120);
        }
        const float down = ldexpf(1.f, -ex);
        uint16_t *prow = part_o + pi * D + 16 * dt0 + 4 * kg;
#pragma unroll
        for (int dt = 0; dt < DT; dt++)
            *reinterpret_cast<uint2 *>(prow + 16 * dt) =
                make_uint2(pack_f16_rne(o[dt][0] * down, o[dt][1] * down), pack_f16_rne(o[dt][2] * down, o[dt][3] * down));
        if (kg == 0) {
#pragma unroll
            for (int qq = 0; qq < 4 / DS; qq++) part_sc[pi * 4 + dpart * (4 / DS) + qq] = ldexpf(1.f, ex);
        }
        if (kg == 0 && dt0 == 0) part_ml[pi] = make_float2(m_run, l_run);
    }
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
            const size_t pi = (size_t)row * nsplit + (s0 + u < nsplit ? s0 + u : nsplit - 1);
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

// Heads per block: enough blocks to fill the chip (about 256) with as many
// heads per block as that allows, so that fewer blocks gather the same rows.
template <int D, int FMT, int HB, int SPLIT>
void launch_mfma_hb(const AttnPlan &p, const void *q, const void *kv, const int32_t *idx, float scale, void *out,
                    float *lse, uint16_t *part_o, float2 *part_ml, float *part_sc, hipStream_t s, const SelHandoff *sel) {
    // two or more waves per head group (each owns a share of the channels)
    // while that stays within 512 threads
    constexpr int DS = HB == 1 ? (D >= 256 ? 4 : 2) : ((HB <= 4 && D >= 128) ? 2 : 1);
    const int npairs = p.B * p.Q * p.nsplit;
    const int NG = p.H / (16 * HB);
    const int blocks = (npairs + 7) / 8 * 8 * NG;
    if (sel)
        hipLaunchKernelGGL((k_attn_mfma<D, FMT, HB, DS, SPLIT, true>), dim3(blocks), dim3(64 * HB * DS), 0, s,
                           static_cast<const uint16_t *>(q), static_cast<const uint8_t *>(kv), p.Q, p.H, p.N, idx, p.k,
                           scale, p.nsplit, npairs, static_cast<uint16_t *>(out), lse, part_o, part_ml, part_sc, *sel);
    else
        hipLaunchKernelGGL((k_attn_mfma<D, FMT, HB, DS, SPLIT, false>), dim3(blocks), dim3(64 * HB * DS), 0, s,
                           static_cast<const uint16_t *>(q), static_cast<const uint8_t *>(kv), p.Q, p.H, p.N, idx, p.k,
                           scale, p.nsplit, npairs, static_cast<uint16_t *>(out), lse, part_o, part_ml, part_sc, SelHandoff{});
}

template <int D, int FMT, int SPLIT>
void launch_mfma_split(const AttnPlan &p, const void *q, const void *kv, const int32_t *idx, float scale, void *out,
                       float *lse, uint16_t *part_o, float2 *part_ml, float *part_sc, hipStream_t s, const SelHandoff *sel) {
    const int64_t pairs = (int64_t)p.B * p.Q * p.nsplit;
    const int hgroups = p.H / 16;
    int hb = hgroups;  // head groups per block
    while (hb > 1 && pairs * (hgroups / hb) < 256) hb /= 2;
    switch (hb) {
        case 1: launch_mfma_hb<D, FMT, 1, SPLIT>(p, q, kv, idx, scale, out, lse, part_o, part_ml, part_sc, s, sel); break;
        case 2: launch_mfma_hb<D, FMT, 2, SPLIT>(p, q, kv, idx, scale, out, lse, part_o, part_ml, part_sc, s, sel); break;
        case 4: launch_mfma_hb<D, FMT, 4, SPLIT>(p, q, kv, idx, scale, out, lse, part_o, part_ml, part_sc, s, sel); break;
        case 8: launch_mfma_hb<D, FMT, 8, SPLIT>(p, q, kv, idx, scale, out, lse, part_o, part_ml, part_sc, s, sel); break;
        default: throw Error(CSA2_EUNSUPPORTED, "matrix-core attention needs H in {16, 32, 64, 128}");
    }
}

template <int D, int FMT>
void launch_mfma(const AttnPlan &p, const void *q, const void *kv, const int32_t *idx, float scale, void *out,
                 float *lse, uint16_t *part_o, float2 *part_ml, float *part_sc, hipStream_t s, const SelHandoff *sel) {
    launch_mfma_split<D, FMT, ATT_SPLIT>(p, q, kv, idx, scale, out, lse, part_o, part_ml, part_sc, s, sel);
}

}  // namespace

AttnPlan attn_plan(int q_dt, int kv_dt, int B, int Q, int H, int D, int64_t N, int k) {
    AttnPlan p{q_dt, kv_dt, B, Q, H, D, N, k, false, 1};
    p.mfma = q_dt == CSA2_BF16 && (kv_dt == CSA2_BF16 || kv_dt == CSA2_FP4) &&
             (H == 16 || H == 32 || H == 64 || H == 128) && (D == 64 || D == 128 || D == 256 || D == 512);
    p.nsplit = p.mfma ? (k + ATT_SPLIT - 1) / ATT_SPLIT : 1;
    return p;
}

bool attn_supported(const AttnPlan &p) {
    if (p.mfma) return (int64_t)p.B * p.Q * p.nsplit * (p.H / 16) + 8 * (p.H / 16) <= INT32_MAX;  // blocks fit an int
    return (p.D + p.k) <= 16384;
}

size_t attn_workspace(const AttnPlan &p) {
    if (!p.mfma || p.nsplit == 1) return 0;
    Carve c(nullptr, 0);
    c.take<uint16_t>((size_t)p.B * p.Q * p.nsplit * p.H * p.D);
    c.take<float2>((size_t)p.B * p.Q * p.nsplit * p.H);
    c.take<float>((size_t)p.B * p.Q * p.nsplit * p.H * 4);
    return c.used;
}

bool attn_handoff_supported(const AttnPlan &p, int64_t nwords) {
    // the bitmap must fit the kernel's LDS tile buffers with room for a band
    return p.mfma && (size_t)((nwords + 3) & ~int64_t(3)) * 4 + 1024 * 16 <= (size_t)2 * ATT_SUB * (p.D + 8) * 2;
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
        if (p.kv_dt == CSA2_FP4) launch_mfma<d, CSA2_FP4>(p, q, kv, idx, scale, out, lse, part_o, part_ml, part_sc, s, sel); \
        else launch_mfma<d, CSA2_BF16>(p, q, kv, idx, scale, out, lse, part_o, part_ml, part_sc, s, sel);                   \
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
