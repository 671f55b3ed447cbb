// Top-k selection for gfx950: exact on given fp32 scores, or certified
// bit-exact against binary64 indexer scores.
//
// "读完这篇，你就搞懂 DeepSeek v4 了", section "闪电索引机制（对应步骤二）": keep
// the k entries with the highest relevance score.  Order (score descending,
// entry index ascending); output the kept indices in ascending order, -1
// padded.  "Recall之王 祭出Reuse", section "把KV Cache压到极致的几把杀手锏": the
// Full layer of the hierarchical indexer also keeps a candidate pool (top-P by
// the same order), inside which Reindex layers select.
//
// Pipeline per query (all kernels run on the caller's stream):
//  1 hist:     the finite scores' range [lo, hi] comes from per-256-slot tile
//              statistics; each 8192-slot chunk builds a 2048-bin histogram of
//              bin(s) = floor((s - lo) * 2048 / (hi - lo)) in LDS.  bin() is
//              monotone in s, computed by one function everywhere.
//  2 find:     sum the chunk histograms, find the bin b* holding the K-th
//              largest score, and by bisection on the float key space the
//              value interval [a, z] of that bin.  Thresholds:
//                IN   = s > z + 2E,   BAND = a - 2E <= s <= z + 2E,   else OUT
//              where E bounds |fp32 score - binary64 score| (E = 0 when the
//              fp32 scores themselves are ranked).  Every IN entry is in the
//              exact top-K and every OUT entry is not.
//  3 classify: write the IN bitmap, count IN, append BAND slots to a list.
//  4 rescore:  (certified only) binary64 score of every BAND entry in the
//              sequential operation order of the definition (lane h: head h's
//              dot product; the products of bf16/fp32 inputs are exact in
//              binary64, so a fused multiply-add equals the rounded product +
//              add).  Up to 32,768 slots and 64 queries, steps 1-4 are one
//              kernel: R replicas of each query's block repeat steps 1-3 and
//              split the band between them.
//  5 band+compact: rank the BAND entries by (exact score, slot) and keep the
//              first K - |IN|; then compact the bitmap in slot order into the
//              ascending index list.
#include "internal.h"

namespace csa2 {

constexpr int NB = 2048;        // histogram bins
constexpr int CH = 8192;        // slots per chunk (256 threads x 32)
constexpr int HIST_CPB = 4;     // chunks per histogram block
constexpr int BANDFAST = 2048;  // largest band ranked by pairwise counting

namespace {

constexpr float NEG_INF = -__builtin_inff();
constexpr float POS_INF = __builtin_inff();

__device__ __forceinline__ int sel_bin(float v, float lo, float inv) {
    float d = v - lo;
    if (!(d > 0.f)) return 0;
    float t = d * inv;
    if (!(t < (float)NB)) return NB - 1;
    return (int)t;
}

// Counts the scores v[] (-inf: no score; finite ones within [lo, hi]) into
// hist[0 .. NB-1] by sel_bin, where inv = NB / (hi - lo) or 0.  When inv is
// finite and > 0 (block-uniform; then hi - lo is finite too, else inv would
// be 0), v - lo lies in [0, hi - lo] and (v - lo) inv is never NaN for a
// finite v: clamped to [-1, NB-1] and truncated it is sel_bin's bin for every
// finite score and -1 for -inf, so no branch per score.  A -inf goes to the
// lane's own spare word hist[NB + lane] (hist holds NB + 64 words): slots with
// no score (past n, outside the candidates, not yet visible) can be most of a
// block's, and one shared spare word would serialize their atomics.
// Otherwise (no finite score, a range of one value or one whose width or
// inverse overflows) each score takes sel_bin itself.
constexpr int NB_SPARE = 64;
template <int NV>
__device__ __forceinline__ void sel_count(const float (&v)[NV], float lo, float inv, uint32_t *hist) {
    if (inv > 0.f && inv <= __FLT_MAX__) {
        const int spare = NB + (int)(threadIdx.x & 63);
#pragma unroll
        for (int i = 0; i < NV; i++) {
            const int bn = (int)fminf(fmaxf((v[i] - lo) * inv, -1.f), (float)(NB - 1));
            atomicAdd(&hist[bn < 0 ? spare : bn], 1u);
        }
    } else {
#pragma unroll
        for (int i = 0; i < NV; i++)
            if (v[i] != NEG_INF) atomicAdd(&hist[sel_bin(v[i], lo, inv)], 1u);
    }
}

__device__ __forceinline__ bool slot_score(const float *scores, const int32_t *cand, int64_t base, int64_t slot,
                                           int64_t n, float &v) {
    if (slot >= n) return false;
    v = scores[base + slot];
    if (v == NEG_INF) return false;
    if (cand && cand[base + slot] < 0) return false;
    return true;
}

template <int NT>
__device__ uint32_t block_sum_u32(uint32_t v, uint32_t *red) {
    v = wave_sum_u32(v);
    const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
    __syncthreads();
    if (lane == 0) red[wave] = v;
    __syncthreads();
    uint32_t t = 0;
    for (int i = 0; i < NT / 64; i++) t += red[i];
    return t;
}

// Exclusive prefix sum over the block (thread order); returns the prefix and
// writes the total.
template <int NT>
__device__ uint32_t block_excl_scan(uint32_t v, uint32_t *buf, uint32_t &total) {
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    uint32_t incl = v;
    for (int o = 1; o < 64; o <<= 1) {
        uint32_t t = __shfl_up(incl, o);
        if (lane >= o) incl += t;
    }
    __syncthreads();
    if (lane == 63) buf[wave] = incl;
    __syncthreads();
    uint32_t before = 0, all = 0;
    for (int i = 0; i < NT / 64; i++) {
        if (i < wave) before += buf[i];
        all += buf[i];
    }
    total = all;
    return before + incl - v;
}

// ---------------------------------------------------- 0: tile statistics
__global__ __launch_bounds__(256) void k_sel_stats(const float *__restrict__ scores, const int32_t *__restrict__ cand,
                                                   int64_t n, int ntiles, TileStat *__restrict__ stats) {
    __shared__ float r_min[4], r_max[4];
    __shared__ uint32_t r_n[4];
    const int bq = blockIdx.y;
    const int64_t base = (int64_t)bq * n;
    float v;
    bool ok = slot_score(scores, cand, base, (int64_t)blockIdx.x * TILE + threadIdx.x, n, v);
    float mn = wave_min(ok ? v : POS_INF), mx = wave_max(ok ? v : NEG_INF);
    uint32_t c = wave_sum_u32(ok ? 1u : 0u);
    const int wave = threadIdx.x >> 6;
    if ((threadIdx.x & 63) == 0) {
        r_min[wave] = mn;
        r_max[wave] = mx;
        r_n[wave] = c;
    }
    __syncthreads();
    if (threadIdx.x == 0) {
        TileStat t;
        t.kmax2 = 0.f;
        t.smin = fminf(fminf(r_min[0], r_min[1]), fminf(r_min[2], r_min[3]));
        t.smax = fmaxf(fmaxf(r_max[0], r_max[1]), fmaxf(r_max[2], r_max[3]));
        t.nvalid = r_n[0] + r_n[1] + r_n[2] + r_n[3];
        stats[(size_t)bq * ntiles + blockIdx.x] = t;
    }
}

// ---------------------------------------------------------------- 1: range
// Per query: the finite scores' range [lo, hi] and count from the tile
// statistics, the bin() parameters into the query record, the query's
// histogram cleared for the chunks' counts, and (certified mode) the score
// error bound from the tiles' largest key norm.
__global__ __launch_bounds__(256) void k_sel_range(const TileStat *__restrict__ stats, int ntiles,
                                                   SelQuery *__restrict__ sq, uint32_t *__restrict__ qhist,
                                                   const double *__restrict__ sumwq, int HI, int dI,
                                                   double *__restrict__ err64, int bf16key) {
    __shared__ float r_min[4], r_max[4], r_k[4];
    __shared__ uint32_t r_n[4];
    const int bq = blockIdx.x, wave = threadIdx.x >> 6;
    float mn = POS_INF, mx = NEG_INF, km = 0.f;
    uint32_t cnt = 0;
    // eight tile records in flight per thread
    for (int t0 = threadIdx.x; t0 < ntiles; t0 += 8 * 256) {
        TileStat st[8];
#pragma unroll
        for (int u = 0; u < 8; u++) {
            const int t = t0 + 256 * u;
            st[u] = stats[(size_t)bq * ntiles + (t < ntiles ? t : t0)];  // past the end: repeat the first
        }
#pragma unroll
        for (int u = 0; u < 8; u++) {
            mn = fminf(mn, st[u].smin);
            mx = fmaxf(mx, st[u].smax);
            km = fmaxf(km, st[u].kmax2);
            if (t0 + 256 * u < ntiles) cnt += st[u].nvalid;
        }
    }
    mn = wave_min(mn);
    mx = wave_max(mx);
    km = wave_max(km);
    cnt = wave_sum_u32(cnt);
    if ((threadIdx.x & 63) == 0) {
        r_min[wave] = mn;
        r_max[wave] = mx;
        r_k[wave] = km;
        r_n[wave] = cnt;
    }
    for (int i = threadIdx.x; i < NB; i += 256) qhist[(size_t)bq * NB + i] = 0;
    __syncthreads();
    if (threadIdx.x == 0) {
        const float lo = fminf(fminf(r_min[0], r_min[1]), fminf(r_min[2], r_min[3]));
        const float hi = fmaxf(fmaxf(r_max[0], r_max[1]), fmaxf(r_max[2], r_max[3]));
        const uint32_t nv = r_n[0] + r_n[1] + r_n[2] + r_n[3];
        const float span = hi - lo;
        sq[bq].lo = lo;
        sq[bq].inv = (nv > 0 && span > 0.f) ? (float)NB / span : 0.f;
        sq[bq].nvalid = (int32_t)nv;
        if (err64) {
            // the score error bound from the largest key norm and the query's sum of w |q|
            const float k2 = fmaxf(fmaxf(r_k[0], r_k[1]), fmaxf(r_k[2], r_k[3]));
            double E = score_bound(sqrt((double)k2 * (1.0 + ldexp(1.0, -10))), sumwq[bq] * (1.0 + ldexp(1.0, -30)),
                                   HI, dI);
            if (bf16key && nv > 0) E = bf16_key_bound(E, fmax(fabs((double)lo), fabs((double)hi)));
            err64[bq] = E;
        }
    }
}

// ---------------------------------------------------------------- 2: hist
// Each 8192-slot chunk counts its scores' bins in LDS (slot CH c + t + 256 i
// in thread t: coalesced loads, all in flight before the counting) and adds
// its nonzero bins to the query's histogram.
template <int CPB>
__global__ __launch_bounds__(256) void k_sel_hist(const float *__restrict__ scores, const int32_t *__restrict__ cand,
                                                  int64_t n, const SelQuery *__restrict__ sq,
                                                  uint32_t *__restrict__ qhist) {
    __shared__ uint32_t hist[NB + NB_SPARE];  // bins, then sel_count's spare words
    const int bq = blockIdx.y;
    for (int i = threadIdx.x; i < NB; i += 256) hist[i] = 0;
    const float lo = sq[bq].lo, inv = sq[bq].inv;
    const int64_t base = (int64_t)bq * n;
    __syncthreads();
    // CPB consecutive chunks per block into one LDS histogram, so that fewer
    // partial histograms are added into the query's (one chunk per block when
    // there are too few chunks to fill the chip otherwise)
    for (int c = 0; c < CPB; c++) {
        const int64_t s0 = ((int64_t)blockIdx.x * CPB + c) * CH + threadIdx.x;
        if (s0 - threadIdx.x >= n) break;
        float v[CH / 256];
#pragma unroll
        for (int i = 0; i < CH / 256; i++) {
            const int64_t sl = s0 + 256 * i;
            v[i] = sl < n ? scores[base + sl] : NEG_INF;
        }
        if (cand) {
#pragma unroll
            for (int i = 0; i < CH / 256; i++) {
                const int64_t sl = s0 + 256 * i;
                if (sl < n && cand[base + sl] < 0) v[i] = NEG_INF;
            }
        }
        sel_count(v, lo, inv, hist);
    }
    __syncthreads();
    for (int i = threadIdx.x; i < NB; i += 256) {
        const uint32_t c = hist[i];
        if (c) atomicAdd(&qhist[(size_t)bq * NB + i], c);
    }
}

__device__ __forceinline__ double thr_lo(float a, double E) {
    if (E > 0.0) return (double)a - 2.0 * E * (1.0 + ldexp(1.0, -20)) - fabs((double)a) * ldexp(1.0, -50);
    return (double)a;
}
__device__ __forceinline__ double thr_hi(float z, double E) {
    if (E > 0.0) return (double)z + 2.0 * E * (1.0 + ldexp(1.0, -20)) + fabs((double)z) * ldexp(1.0, -50);
    return (double)z;
}

// Order-preserving key of the bin edge: defined with the one-block path.
__device__ uint32_t edge_key(uint32_t lk, uint32_t hk, int target, float lo, float inv);

// ---------------------------------------------------------------- 3: find
__global__ __launch_bounds__(256) void k_sel_find(const uint32_t *__restrict__ qhist, int K0, int K1,
                                                  const double *__restrict__ ebound, SelQuery *__restrict__ sq) {
    __shared__ uint32_t cum[NB + 1];
    __shared__ int bstar;
    __shared__ uint32_t edge[2];
    const int bq = blockIdx.x;
    // per-thread 8 consecutive bins of the query's histogram
    uint32_t h[8];
    uint32_t local = 0;
#pragma unroll
    for (int i = 0; i < 8; i++) {
        h[i] = qhist[(size_t)bq * NB + threadIdx.x * 8 + i];
        local += h[i];
    }
    // suffix sums: cum[b] = number of finite scores in bins >= b
    __shared__ uint32_t tot[4];
    uint32_t all;
    const uint32_t before = block_excl_scan<256>(local, tot, all);
    uint32_t run = all - before - local;  // finite scores in the bins of later threads
    for (int i = 7; i >= 0; i--) {
        run += h[i];
        cum[threadIdx.x * 8 + i] = run;
    }
    if (threadIdx.x == 0) cum[NB] = 0;
    __syncthreads();
    const SelQuery q = sq[bq];
    const double E = ebound ? ebound[bq] : 0.0;
    for (int tgt = 0; tgt < 2; tgt++) {
        const int K = tgt == 0 ? K0 : K1;
        if (K <= 0) continue;
        if (threadIdx.x == 0) bstar = -1;
        __syncthreads();
        if (q.nvalid > K) {
            for (int i = 0; i < 8; i++) {
                int b = threadIdx.x * 8 + i;
                if (cum[b] >= (uint32_t)K && cum[b + 1] < (uint32_t)K) bstar = b;
            }
        }
        __syncthreads();
        // [a, z] = the float values >= lo whose bin is b* (bin() is monotone):
        // wave 0 finds the lower edge a, wave 1 the upper edge z
        if (bstar >= 0 && threadIdx.x < 128) {
            const int wave = threadIdx.x >> 6;
            const uint32_t lk = fkey(q.lo), hk = 0xff7fffffu;  // hk: key of the largest finite float
            uint32_t kk = hk;
            if (wave == 0) kk = edge_key(lk, hk, bstar, q.lo, q.inv);
            else if (bstar + 1 < NB) kk = edge_key(lk, hk, bstar + 1, q.lo, q.inv) - 1;
            if ((threadIdx.x & 63) == 0) edge[wave] = kk;
        }
        __syncthreads();
        if (threadIdx.x == 0) {
            SelTarget t;
            t.K = K;
            t.in_cnt = 0;
            t.band_cnt = 0;
            t.pad = 0;
            if (bstar < 0) {  // every finite score is kept
                t.lo = -__builtin_inf();
                t.hi = -__builtin_inf();
            } else {
                t.lo = thr_lo(fkey_inv(edge[0]), E);
                t.hi = thr_hi(fkey_inv(edge[1]), E);
            }
            sq[bq].t[tgt] = t;
        }
        __syncthreads();
    }
}

// ------------------------------------------------------------ 4: classify
// Largest float <= d and smallest float >= d (d finite or -inf).
__device__ __forceinline__ float f32_down(double d) {
    float f = (float)d;
    if ((double)f > d) f = nextafterf(f, NEG_INF);
    return f;
}
__device__ __forceinline__ float f32_up(double d) {
    float f = (float)d;
    if ((double)f < d) f = nextafterf(f, POS_INF);
    return f;
}

// A block takes CLS_WPT x 256 consecutive bitmap words; thread t holds words
// w0 + t + 256 u (slots 32 w .. 32 w + 31, with 16-byte loads where a word is
// whole), so its comparisons against the thresholds are those words' IN and
// BAND bits.  Thresholds are the binary64 bounds rounded outward to floats.
// The counts meet per block first and reach the query record with one atomic
// update per block and target: the records are shared by every block of a
// query, and per-wave updates of one address queue up.
constexpr int CLS_WPT_MAX = 4;  // words per thread (1 when there are too few words to fill the chip otherwise)

__device__ __forceinline__ void load_word_scores(const float *sp, const int32_t *cp, int64_t s0, int64_t n,
                                                 float *v) {
    if (s0 + 32 <= n && ((reinterpret_cast<uintptr_t>(sp) | reinterpret_cast<uintptr_t>(cp)) & 15) == 0) {
#pragma unroll
        for (int i = 0; i < 32; i += 4) {
            const f32x4 q4 = *reinterpret_cast<const f32x4 *>(sp + s0 + i);
            v[i] = q4[0], v[i + 1] = q4[1], v[i + 2] = q4[2], v[i + 3] = q4[3];
        }
        if (cp) {
#pragma unroll
            for (int i = 0; i < 32; i += 4) {
                const u32x4 c4 = *reinterpret_cast<const u32x4 *>(cp + s0 + i);
#pragma unroll
                for (int e = 0; e < 4; e++)
                    if ((int32_t)c4[e] < 0) v[i + e] = NEG_INF;
            }
        }
    } else {
#pragma unroll
        for (int i = 0; i < 32; i++) {
            const int64_t sl = s0 + i;
            v[i] = sl < n ? sp[sl] : NEG_INF;
            if (cp && sl < n && cp[sl] < 0) v[i] = NEG_INF;
        }
    }
}

template <int CLS_WPT>
__global__ __launch_bounds__(256) void k_sel_classify(const float *__restrict__ scores,
                                                      const int32_t *__restrict__ cand, int64_t n, int ntgt,
                                                      SelQuery *__restrict__ sq, uint32_t *__restrict__ bitmap,
                                                      int64_t nwords, int32_t *__restrict__ band, int64_t band_cap) {
    __shared__ uint32_t w_in[4], w_nb[4];
    __shared__ int32_t base_sh;
    const int bq = blockIdx.y, lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const int64_t wbase0 = (int64_t)blockIdx.x * (256 * CLS_WPT) + threadIdx.x;
    const float *sp = scores + (int64_t)bq * n;
    const int32_t *cp = cand ? cand + (int64_t)bq * n : nullptr;
    float v[CLS_WPT][32];
#pragma unroll
    for (int u = 0; u < CLS_WPT; u++) load_word_scores(sp, cp, (wbase0 + 256 * u) * 32, n, v[u]);
    for (int tgt = 0; tgt < ntgt; tgt++) {
        const SelTarget t = sq[bq].t[tgt];
        // IN: x > hi <=> x > f_hi;  BAND: x >= lo <=> x >= f_lo (x a float); -inf
        // (no score) is neither, since f_lo is made finite
        const float f_hi = f32_down(t.hi), f_lo = fmaxf(f32_up(t.lo), -__FLT_MAX__);
        uint32_t bandw[CLS_WPT], nin = 0, nb = 0;
#pragma unroll
        for (int u = 0; u < CLS_WPT; u++) {
            const int64_t word = wbase0 + 256 * u;
            uint32_t in = 0, bm = 0;
#pragma unroll
            for (int i = 0; i < 32; i++) {
                in |= (v[u][i] > f_hi ? 1u : 0u) << i;
                bm |= (v[u][i] <= f_hi && v[u][i] >= f_lo ? 1u : 0u) << i;
            }
            if (word < nwords) bitmap[((size_t)tgt * gridDim.y + bq) * nwords + word] = in;
            bandw[u] = bm;
            nin += (uint32_t)__builtin_popcount(in);
            nb += (uint32_t)__builtin_popcount(bm);
        }
        const uint32_t incl = wave_incl_scan_u32(nb);
        const uint32_t wnin = wave_sum_u32(nin);
        if (lane == 63) w_nb[wave] = incl;
        if (lane == 0) w_in[wave] = wnin;
        __syncthreads();
        if (threadIdx.x == 0) {
            const uint32_t bin = w_in[0] + w_in[1] + w_in[2] + w_in[3];
            const uint32_t bnb = w_nb[0] + w_nb[1] + w_nb[2] + w_nb[3];
            if (bin) atomicAdd(&sq[bq].t[tgt].in_cnt, (int32_t)bin);
            base_sh = bnb ? atomicAdd(&sq[bq].t[tgt].band_cnt, (int32_t)bnb) : 0;
        }
        __syncthreads();
        int32_t pos = base_sh + (int32_t)(incl - nb);
        for (int w = 0; w < wave; w++) pos += (int32_t)w_nb[w];
        int32_t *dst = band + ((size_t)tgt * gridDim.y + bq) * band_cap;
#pragma unroll
        for (int u = 0; u < CLS_WPT; u++) {
            const int64_t s0 = (wbase0 + 256 * u) * 32;
            for (uint32_t m = bandw[u]; m; m &= m - 1) dst[pos++] = (int32_t)(s0 + __builtin_ctz(m));
        }
        __syncthreads();  // w_in, w_nb and base_sh are reused by the next target
    }
}

// ------------------------------------------------- shared finishing steps

__device__ __forceinline__ uint32_t load_word(const uint32_t *p) {
    return __hip_atomic_load(p, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}


// Smallest order-preserving float key in [L, R] whose bin is >= target
// (R + 1 if none), by a 64-way search run by one whole wave.
__device__ uint32_t wave_search_bin(uint32_t L, uint32_t R, int target, float lo, float inv) {
    const int lane = threadIdx.x & 63;
    uint64_t lo64 = L, hi64 = (uint64_t)R + 1;  // answer in [lo64, hi64]
    while (hi64 - lo64 > 0) {
        const uint64_t span = hi64 - lo64;
        const uint64_t step = span / 64 + 1;
        const uint64_t p = lo64 + (uint64_t)lane * step;
        // points at or beyond hi64 count as satisfying (hi64 is the answer when
        // nothing below it does), so the ballot is monotone in the lane:
        // false ... false true ... true
        const bool t = p >= hi64 || sel_bin(fkey_inv((uint32_t)p), lo, inv) >= target;
        const uint64_t bal = __ballot(t);
        const int f = bal ? __builtin_ctzll(bal) : 64;
        if (f == 0) {
            hi64 = lo64;  // p_0 = lo64 satisfies it
        } else {
            // p_{f-1} < hi64 fails, so the answer is in (p_{f-1}, min(p_f, hi64)]
            const uint64_t pf1 = lo64 + (uint64_t)(f - 1) * step;
            const uint64_t pf = lo64 + (uint64_t)f * step;
            lo64 = pf1 + 1;
            if (f < 64 && pf < hi64) hi64 = pf;
        }
    }
    return (uint32_t)lo64;
}


// The r best of nb <= 2 NT band entries by (key descending, slot ascending),
// set in the bitmap: a radix select of the r-th largest 96-bit composite
// (key, ~slot), one byte per pass from the top.  Composites are unique (slots
// are), so exactly r entries are at or above it.  Entries live in registers
// (two per thread); `hist` is LDS scratch of at least 258 words.
template <int NT>
__device__ void radix_pick(uint32_t *bm, int32_t nb, int32_t r, const uint64_t (&key)[2], const int32_t (&slot)[2],
                           uint32_t *hist) {
    const int tid = threadIdx.x, lane = tid & 63;
    bool live[2], take[2];
#pragma unroll
    for (int e = 0; e < 2; e++) {
        live[e] = tid + NT * e < nb;
        take[e] = false;
    }
    uint32_t need = (uint32_t)r;
    auto digit = [&](int e, int p) -> uint32_t {  // byte p of the composite, 11 = most significant
        return p >= 4 ? (uint32_t)(key[e] >> (8 * (p - 4))) & 0xffu : (~(uint32_t)slot[e] >> (8 * p)) & 0xffu;
    };
    // bytes above the highest one in which two entries differ select nothing:
    // OR of every composite XOR entry 0's, reduced per wave, then in LDS
    if (tid == 0) {
        hist[260] = (uint32_t)key[0];
        hist[261] = (uint32_t)(key[0] >> 32);
        hist[262] = (uint32_t)slot[0];
        hist[263] = hist[264] = hist[265] = 0;
    }
    __syncthreads();
    const uint64_t k0 = (uint64_t)hist[260] | ((uint64_t)hist[261] << 32);
    const uint32_t s0 = hist[262];
    uint32_t dx[3] = {0u, 0u, 0u};
#pragma unroll
    for (int e = 0; e < 2; e++)
        if (live[e]) {
            dx[0] |= (uint32_t)(key[e] ^ k0);
            dx[1] |= (uint32_t)((key[e] ^ k0) >> 32);
            dx[2] |= (uint32_t)slot[e] ^ s0;
        }
#pragma unroll
    for (int i = 0; i < 3; i++) {
        for (int o = 32; o > 0; o >>= 1) dx[i] |= (uint32_t)__shfl_xor((int)dx[i], o);
        if (lane == 0 && dx[i]) atomicOr(&hist[263 + i], dx[i]);
    }
    __syncthreads();
    const uint32_t kxl = hist[263], kxh = hist[264], sx = hist[265];
    const int ptop = kxh ? 8 + (31 - __builtin_clz(kxh)) / 8
                         : kxl ? 4 + (31 - __builtin_clz(kxl)) / 8 : sx ? (31 - __builtin_clz(sx)) / 8 : 0;
    for (int p = ptop; p >= 0; p--) {
        for (int i = tid; i < 256; i += NT) hist[i] = 0;
        __syncthreads();
#pragma unroll
        for (int e = 0; e < 2; e++)
            if (live[e]) atomicAdd(&hist[digit(e, p)], 1u);
        __syncthreads();
        if (tid < 64) {
            // suffix counts over the 256 digits, lane l holding digits 4 (63 - l) .. +3
            uint32_t h[4], loc = 0;
#pragma unroll
            for (int j = 0; j < 4; j++) {
                h[j] = hist[4 * (63 - lane) + j];
                loc += h[j];
            }
            const uint32_t incl = wave_incl_scan_u32(loc);  // counts of digits >= 4 (63 - l)
            uint32_t above = incl - loc;                     // counts of digits > 4 (63 - l) + 3
#pragma unroll
            for (int j = 3; j >= 0; j--) {
                if (above < need && above + h[j] >= need) {
                    hist[256] = 4 * (63 - lane) + j;
                    hist[257] = need - above;
                    hist[258] = h[j];
                }
                above += h[j];
            }
        }
        __syncthreads();
        const uint32_t d = hist[256];
        need = hist[257];
        const bool done = hist[258] == need;  // every entry left in digit d is taken
#pragma unroll
        for (int e = 0; e < 2; e++)
            if (live[e]) {
                const uint32_t g = digit(e, p);
                take[e] |= g > d || (done && g == d);
                live[e] = !done && g == d;
            }
        __syncthreads();  // hist is cleared by the next pass
        if (done) break;
    }
#pragma unroll
    for (int e = 0; e < 2; e++)
        if (take[e] || live[e]) atomicOr(&bm[slot[e] >> 5], 1u << (slot[e] & 31));
}

// Write the set bits of the bitmap `bm` (LDS or global) in slot order as the
// ascending index list dst[0, K) (mapped through cand_q when given, -1
// padded) and the count.  Each wave sweeps 2048 consecutive words per round
// with coalesced 16-byte loads (lane l holds words 4 l .. 4 l + 3 of each
// 256-word group); positions come from wave scans of the popcounts and one
// exchange of the wave totals.  The list is staged in LDS (out_cap ints) when
// it fits, for coalesced writes; sweeping stops once K entries are placed.
template <int NT>
__device__ void compact_bits(const uint32_t *bm, int64_t nwords, int32_t K, const int32_t *cand_q, int32_t *dst,
                             int32_t *count_dst, int32_t *out_lds, int out_cap, uint32_t *red) {
    constexpr int NW = NT / 64, G = 4;
    constexpr int64_t WSPAN = 256 * G, SPAN = WSPAN * NW;
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const bool staged = K <= out_cap;
    const bool vec = (reinterpret_cast<uintptr_t>(bm) & 15) == 0;
    uint32_t base = 0;
    for (int64_t c0 = 0; c0 < nwords && base < (uint32_t)K; c0 += SPAN) {
        const int64_t wb = c0 + wave * WSPAN + 4 * lane;
        uint32_t v[G][4];
#pragma unroll
        for (int g = 0; g < G; g++) {
            const int64_t w = wb + 256 * g;
            if (vec && w + 3 < nwords) {
                const u32x4 t = *reinterpret_cast<const u32x4 *>(bm + w);
#pragma unroll
                for (int j = 0; j < 4; j++) v[g][j] = t[j];
            } else {
#pragma unroll
                for (int j = 0; j < 4; j++) v[g][j] = w + j < nwords ? bm[w + j] : 0u;
            }
        }
        uint32_t ex[G], gt[G], wt = 0;
#pragma unroll
        for (int g = 0; g < G; g++) {
            const uint32_t c = __builtin_popcount(v[g][0]) + __builtin_popcount(v[g][1]) +
                               __builtin_popcount(v[g][2]) + __builtin_popcount(v[g][3]);
            const uint32_t incl = wave_incl_scan_u32(c);
            ex[g] = incl - c;
            gt[g] = (uint32_t)__builtin_amdgcn_readlane((int)incl, 63);
            wt += gt[g];
        }
        if (lane == 0) red[wave] = wt;
        __syncthreads();
        uint32_t pos0 = base, all = 0;
        for (int i = 0; i < NW; i++) {
            const uint32_t t = red[i];
            if (i < wave) pos0 += t;
            all += t;
        }
        __syncthreads();  // red is rewritten next round
#pragma unroll
        for (int g = 0; g < G; g++) {
            uint32_t pos = pos0 + ex[g];
#pragma unroll
            for (int j = 0; j < 4; j++) {
                uint32_t bits = v[g][j];
                while (bits) {
                    const int i = __builtin_ctz(bits);
                    bits &= bits - 1;
                    if (pos < (uint32_t)K) {
                        const int64_t sl = (wb + 256 * g + j) * 32 + i;
                        const int32_t val = cand_q ? cand_q[sl] : (int32_t)sl;
                        if (staged) out_lds[pos] = val;
                        else dst[pos] = val;
                    }
                    pos++;
                }
            }
            pos0 += gt[g];
        }
        base += all;
    }
    const uint32_t kept = base < (uint32_t)K ? base : (uint32_t)K;
    if (staged) {
        __syncthreads();
        for (int32_t i = threadIdx.x; i < K; i += NT) dst[i] = i < (int32_t)kept ? out_lds[i] : -1;
    } else {
        for (int32_t i = kept + threadIdx.x; i < K; i += NT) dst[i] = -1;
    }
    if (count_dst && threadIdx.x == 0) *count_dst = (int32_t)kept;
    __syncthreads();
}

// Pick the best r = K - |IN| BAND entries of one target by (exact score
// descending, slot ascending) and set their bits in the LDS bitmap `bm`, then
// compact the bitmap in slot order into the ascending index list (-1 padded).
// Keys: binary64 band scores when `bs` is given, else the fp32 scores.  The
// output is staged in LDS (out_cap ints) when it fits, for coalesced writes.
template <int NT>
__device__ void finish_target(uint32_t *bm, int64_t nwords, int64_t n, int32_t K, int32_t in_cnt, int32_t nb,
                              const int32_t *list, const double *bs, const float *scores_q,
                              const int32_t *cand_q, int32_t *dst, int32_t *count_dst, uint64_t *key_lds,
                              int32_t *slot_lds, int32_t *out_lds, int out_cap, uint32_t *red,
                              bool preloaded = false, bool bm_global = false) {
    const int32_t r = K - in_cnt;
    auto exact_key = [&](int32_t i) -> uint64_t { return dkey(bs ? bs[i] : (double)scores_q[list[i]]); };
    if (r > 0 && nb > 0 && r < nb && nb > 256 && nb <= 2 * NT) {
        // many entries: radix select, O(nb) work per pass instead of O(nb^2) comparisons
        uint64_t kk[2];
        int32_t ss[2];
#pragma unroll
        for (int e = 0; e < 2; e++) {
            const int32_t i = threadIdx.x + NT * e;
            const int32_t ii = i < nb ? i : nb - 1;
            kk[e] = preloaded ? key_lds[ii] : exact_key(ii);
            ss[e] = preloaded ? slot_lds[ii] : list[ii];
        }
        __syncthreads();  // the LDS entries are read before key_lds becomes the histogram
        radix_pick<NT>(bm, nb, r, kk, ss, reinterpret_cast<uint32_t *>(key_lds));
    } else if (r > 0 && nb > 0) {
        if (nb <= BANDFAST) {
            if (!preloaded)
                for (int32_t i = threadIdx.x; i < nb; i += NT) {
                    key_lds[i] = exact_key(i);
                    slot_lds[i] = list[i];
                }
            __syncthreads();
            for (int32_t i = threadIdx.x; i < nb; i += NT) {
                const uint64_t ki = key_lds[i];
                const int32_t si = slot_lds[i];
                int32_t rank = 0;
                int32_t j0 = 0;
                for (; j0 + 16 <= nb; j0 += 16) {
                    uint64_t kk[16];
                    int32_t ss[16];
#pragma unroll
                    for (int u = 0; u < 16; u++) {
                        kk[u] = key_lds[j0 + u];
                        ss[u] = slot_lds[j0 + u];
                    }
#pragma unroll
                    for (int u = 0; u < 16; u++) rank += (int)((kk[u] > ki) | ((kk[u] == ki) & (ss[u] < si)));
                }
                for (; j0 < nb; j0++) {
                    const uint64_t kj = key_lds[j0];
                    rank += (int)((kj > ki) | ((kj == ki) & (slot_lds[j0] < si)));
                }
                if (rank < r) atomicOr(&bm[si >> 5], 1u << (si & 31));
            }
        } else {
            // bisection on the key for the r-th best, then on the slot among ties
            uint64_t L = 0, R = ~0ull;
            while (L < R) {
                const uint64_t M = L + (R - L) / 2 + 1;
                uint32_t c = 0;
                for (int32_t i = threadIdx.x; i < nb; i += NT) c += exact_key(i) >= M;
                c = block_sum_u32<NT>(c, red);
                if (c >= (uint32_t)r) L = M;
                else R = M - 1;
            }
            const uint64_t tau = L;
            uint32_t gt = 0;
            for (int32_t i = threadIdx.x; i < nb; i += NT) gt += exact_key(i) > tau;
            gt = block_sum_u32<NT>(gt, red);
            const uint32_t need = (uint32_t)r - gt;
            int64_t SL = 0, SR = n - 1;
            while (SL < SR) {
                const int64_t M = SL + (SR - SL) / 2;
                uint32_t c = 0;
                for (int32_t i = threadIdx.x; i < nb; i += NT) c += (exact_key(i) == tau) && (list[i] <= M);
                c = block_sum_u32<NT>(c, red);
                if (c >= need) SR = M;
                else SL = M + 1;
            }
            for (int32_t i = threadIdx.x; i < nb; i += NT) {
                const uint64_t k = exact_key(i);
                const int32_t sl = list[i];
                if (k > tau || (k == tau && sl <= SL)) atomicOr(&bm[sl >> 5], 1u << (sl & 31));
            }
        }
    }
    // the picks are complete and visible before the bitmap is read: LDS
    // atomics by the barrier alone; global ones (a bitmap too large for LDS)
    // after a device fence, which costs microseconds and is skipped otherwise
    if (bm_global) __threadfence();
    __syncthreads();
    compact_bits<NT>(bm, nwords, K, cand_q, dst, count_dst, out_lds, out_cap, red);
}

// ------------------------------------------------------ one-block path
// One 1024-thread block per query keeps its n <= 32768 scores in registers
// (thread t holds slots 32 t .. 32 t + 31, so its 32 comparisons against a
// threshold are bitmap word t, built without any cross-lane step).  With the score range known from
// the indexer's tile statistics (else from the scores), the 2048-bin
// histogram is built from registers, the bin edges of the K-th largest come
// from a 64-way search in a narrow window around their estimate, and the
// classification compares in fp32 against thresholds rounded outward.  Exact
// mode also picks the band and compacts (one launch); certified mode hands
// the IN bitmap and the band list on.
constexpr int ONE_NT = 1024;
constexpr int64_t ONE_N = 32768;
constexpr int ONE_SPT = (int)(ONE_N / ONE_NT);
constexpr int ONE_OUT = 8192;  // output entries staged in LDS
static_assert(ONE_SPT == 32, "a thread's slots form one bitmap word");

// ----------------------------------------------------------------- rescore
// One wave per BAND entry (both targets' lists back to back), no staging:
// lane h loads query head h's row and the key row (the same address in every
// lane) with 16-byte loads into registers, and computes head h's dot product
// in the definition's order d = 0, 1, ... (products of bf16/fp32 inputs are
// exact in binary64, so fma = rounded product + add); t_h = w_h * ReLU(d_h)
// is rounded on its own, and lane 0 sums t_0, t_1, ... from +0.0 out of LDS.
// Idle blocks exit at once.
constexpr int RS_NT = 256;
constexpr int RS_VB = 16;      // 16-byte vectors per row batch

struct RescoreKArgs {
    const void *qI;
    int dt;
    int kfp4;  // key rows in FP4 (queries bf16)
    const float *w;
    const void *kI;
    int Q, HI, dI;
    int64_t N;
    const int32_t *cand;
    int64_t n;
    int ntgt;
    const SelQuery *sq;
    const int32_t *band;
    double *band_score;
    int64_t band_cap;
    int bf16key;  // store the scores rounded to bfloat16 (the ranked value)
};

// Running binary64 dot over one 16-byte vector of each row.
template <bool F32>
__device__ __forceinline__ double dot_vec(double acc, u32x4 q, u32x4 k) {
#pragma clang fp contract(off)
    if constexpr (F32) {
#pragma unroll
        for (int e = 0; e < 4; e++) acc = __builtin_fma((double)__uint_as_float(q[e]), (double)__uint_as_float(k[e]), acc);
    } else {
#pragma unroll
        for (int e = 0; e < 4; e++) {
            acc = __builtin_fma((double)__uint_as_float(q[e] << 16), (double)__uint_as_float(k[e] << 16), acc);
            acc = __builtin_fma((double)__uint_as_float(q[e] & 0xffff0000u), (double)__uint_as_float(k[e] & 0xffff0000u),
                                acc);
        }
    }
    return acc;
}

constexpr int RS_EPW = 2;                       // entries per wave
constexpr int RS_EPB = RS_EPW * (RS_NT / 64);  // entries per block
constexpr int RS_ROWB = 512;                    // longest key row staged (bytes)
constexpr int RS_MAXD = RS_ROWB / 2;            // longest staged row in elements
constexpr int RS_QS = RS_ROWB / 16 + 1;        // LDS stride of a staged query row in 16-byte vectors (padded)


// Piece c of key row `row` as exact binary64 values: 16 bytes of bf16 or
// fp32 values, or (FP4 rows) 8 channels from 4 code bytes and their E4M3
// scale byte.
template <bool F32>
__device__ __forceinline__ void rs_stage_piece(const void *kI, int kfp4, size_t row, int dI, int c, double *dst) {
    constexpr int ESZ = F32 ? 4 : 2;
    constexpr int EPV = 16 / ESZ;  // elements per 16-byte vector
    if (!F32 && kfp4) {
        const uint8_t *krow = static_cast<const uint8_t *>(kI) + row * (size_t)(dI / 2 + dI / 16);
        const uint32_t cw = *reinterpret_cast<const uint32_t *>(krow + 4 * c);
        const uint32_t sb = krow[dI / 2 + c / 2];
        const uint32_t se = (sb >> 3) & 15u, sm = sb & 7u;
        double sc = se ? (double)(8u + sm) * __builtin_ldexp(1.0, (int)se - 10) : (double)sm * 0x1p-9;
        if ((sb & 0x7fu) == 0x7fu) sc = 448.0;  // the E4M3 NaN code saturates
        if (sb & 0x80u) sc = -sc;
#pragma unroll
        for (int x = 0; x < 8; x++) {
            const uint32_t cd = (cw >> (4 * x)) & 15u;
            const uint32_t ce = (cd >> 1) & 3u, mb = cd & 1u;
            const double mag = ce ? (1.0 + 0.5 * mb) * __builtin_ldexp(1.0, (int)ce - 1) : 0.5 * mb;
            dst[x] = ((cd & 8u) ? -mag : mag) * sc;
        }
    } else {
        const u32x4 kv = reinterpret_cast<const u32x4 *>(static_cast<const char *>(kI) + row * dI * ESZ)[c];
#pragma unroll
        for (int x = 0; x < EPV; x++) {
            const uint32_t kw = kv[F32 ? x : x >> 1];
            dst[x] = (double)__uint_as_float(F32 ? kw : ((x & 1) ? (kw & 0xffff0000u) : (kw << 16)));
        }
    }
}

// Binary64 scores of the staged entries ew .. ew + RS_EPW - 1 of query bq
// (their key rows in krow as binary64, the first 64 heads' query rows in
// qsh; heads past 64 read from memory): lane h runs head h's dot products
// of the RS_EPW entries as independent chains in the definition's order
// d = 0, 1, ..., t_h = w_h * ReLU(d_h) goes through the wave's LDS rows tl,
// and lane e < RS_EPW sums entry e's terms in head order from +0.0.
// Returns lane e's score (not rounded to a key), 0 in the other lanes.
// QCH query vectors are held at a time.
template <bool F32, int QCH = 16>
__device__ double rs_wave_scores(const void *qI, const float *w, int bq, int HI, int dI,
                                 const u32x4 (*qsh)[RS_QS], const double (*krow_lds)[RS_MAXD], int ew,
                                 double (*tl)[64]) {
#pragma clang fp contract(off)
    constexpr int ESZ = F32 ? 4 : 2;
    constexpr int EPV = 16 / ESZ;
    const int lane = threadIdx.x & 63;
    const int nvec = dI * ESZ / 16;
    double sc = 0.0;  // lane e < RS_EPW: running score of entry ew + e
    for (int h0 = 0; h0 < HI; h0 += 64) {
        const int h = h0 + lane;
        const int hc = h < HI ? h : HI - 1;  // idle lanes recompute the last head, unused
        const u32x4 *qrow = reinterpret_cast<const u32x4 *>(static_cast<const char *>(qI) +
                                                            ((size_t)bq * HI + hc) * dI * ESZ);
        const double wh = (double)w[(size_t)bq * HI + hc];
        double dot[RS_EPW];
#pragma unroll
        for (int e = 0; e < RS_EPW; e++) dot[e] = 0.0;
        for (int v0 = 0; v0 < nvec; v0 += QCH) {
            u32x4 qv[QCH];
            if (h0 == 0) {
#pragma unroll
                for (int u = 0; u < QCH; u++)
                    if (v0 + u < nvec) qv[u] = qsh[lane][v0 + u];
            } else {
#pragma unroll
                for (int u = 0; u < QCH; u++)
                    if (v0 + u < nvec) qv[u] = qrow[v0 + u];
            }
#pragma unroll
            for (int u = 0; u < QCH; u++) {
                if (v0 + u >= nvec) break;
#pragma unroll
                for (int x = 0; x < EPV; x += 2) {
                    const uint32_t qw0 = qv[u][F32 ? x : x >> 1];
                    const uint32_t qw1 = qv[u][F32 ? x + 1 : x >> 1];
                    const double qd0 = (double)__uint_as_float(F32 ? qw0 : (qw0 << 16));
                    const double qd1 = (double)__uint_as_float(F32 ? qw1 : (qw1 & 0xffff0000u));
#pragma unroll
                    for (int e = 0; e < RS_EPW; e++) {
                        const double2 k2 = *reinterpret_cast<const double2 *>(&krow_lds[ew + e][(v0 + u) * EPV + x]);
                        dot[e] = __builtin_fma(qd0, k2.x, dot[e]);
                        dot[e] = __builtin_fma(qd1, k2.y, dot[e]);
                    }
                }
            }
        }
#pragma unroll
        for (int e = 0; e < RS_EPW; e++) tl[e][lane] = h < HI ? wh * (dot[e] > 0.0 ? dot[e] : 0.0) : 0.0;
        __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
        __builtin_amdgcn_wave_barrier();
        __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
        if (lane < RS_EPW) {
            // head terms t_h0, t_h0+1, ... added in order (read 16 at a time);
            // lanes past the last head hold +0.0, and sc + 0.0 == sc (sc is
            // never -0.0: it starts at +0.0 and a round-to-nearest sum is
            // -0.0 only if both addends are)
            const int hn = HI - h0 < 64 ? HI - h0 : 64;
            for (int c0 = 0; c0 < hn; c0 += 16) {
                double tv[16];
#pragma unroll
                for (int i = 0; i < 16; i++) tv[i] = tl[lane][c0 + i];
#pragma unroll
                for (int i = 0; i < 16; i++) sc = sc + tv[i];
            }
        }
        __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
        __builtin_amdgcn_wave_barrier();
        __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
    }
    return lane < RS_EPW ? sc : 0.0;
}

struct OneArgs {
    const float *scores;
    const int32_t *cand;
    int64_t n;
    int K[2];
    int ntgt;
    // certified: range and error bound inputs from the indexer
    const TileStat *stats;
    int ntiles;
    const double *sumwq;
    int HI, dI;
    // exact-mode outputs
    int32_t *out0, *count0, *out1;
    // certified hand-off
    SelQuery *sq;
    uint32_t *bitmap;
    int64_t nwords;
    int32_t *band;
    int64_t band_cap;
    int32_t *in_list;  // certified, nullable: target 0's IN entries in ascending order, [BQ][K0]
    int bf16key;       // certified: the ranked value is the score rounded to bfloat16
    // certified, nullable qI: the band's binary64 scores computed here, the
    // band split over the gridDim.y replicas of each query's block (else the
    // rescoring kernel computes them)
    const void *qI;
    int rs_f32, kfp4;
    const float *w;
    const void *kI;
    int Q;
    int64_t N;
    double *band_score;
};

constexpr int OR_CH = RS_EPW * (ONE_NT / 64);  // band entries a replica rescores per round
constexpr int OR_QPT = 64 * (RS_ROWB / 16) / ONE_NT;  // query-row vectors per thread (heads 0 .. 63)

// Exclusive prefix sum over the block's threads in thread order, and the
// block's total; red holds NT / 64 words and is free again on return.
template <int NT>
__device__ __forceinline__ uint32_t block_excl_scan_u32(uint32_t c, uint32_t *red, uint32_t &total) {
    const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
    const uint32_t inc = wave_incl_scan_u32(c);
    if (lane == 63) red[wave] = inc;
    __syncthreads();
    uint32_t pre = 0, tot = 0;
#pragma unroll
    for (int i = 0; i < NT / 64; i++) {
        const uint32_t r = red[i];
        pre += i < wave ? r : 0u;
        tot += r;
    }
    __syncthreads();
    total = tot;
    return pre + inc - c;
}

// The band rescoring inside the one-block selection, with F * ONE_NT / 64
// replicas of each query's block (F = 1, 2 or 4): every replica classified
// the same slots, so each holds the same band lists (target 0's, then target
// 1's, each in slot order, at positions from the block scan).  Replica r
// rescores the band entries of lanes r % F of F equal lane ranges of wave
// r / F (2048 / F slots): that wave lists them in LDS
// (slot, target, position) by a wave scan, the key rows are staged in LDS as
// binary64 OR_CH at a time, and each wave computes RS_EPW entries' scores in
// the definition's order (rs_wave_scores), as the rescoring kernel does.
// The first 64 heads' query rows are in qsh already.
template <bool F32>
__device__ void one_rescore(const OneArgs &a, int bq, int rep, int s0, uint32_t kw0, uint32_t kw1, int32_t kp0,
                            int32_t kp1, uint32_t *ents, int32_t *nent_sh, double (*krow)[RS_MAXD],
                            u32x4 (*qsh)[RS_QS], double (*tl)[RS_EPW][64]) {
    constexpr int ESZ = F32 ? 4 : 2;
    constexpr int EPV = 16 / ESZ;
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int b = bq / a.Q;
    const int nvec = a.dI * ESZ / 16;
    const size_t row0 = (size_t)bq * a.band_cap, row1 = ((size_t)gridDim.x + bq) * a.band_cap;
    // replica rep takes the band entries of lanes [l0, l0 + 64 / F) of wave
    // rep / F (F = replicas per wave, gridDim.y / 16): their slots
    const int F = max(1, (int)gridDim.y / (ONE_NT / 64));
    const int l0 = (rep % F) * (64 / F);
    if (wave == rep / F) {
        // entry: slot | target << 15 | position << 16 (slots and positions < 32,768)
        const bool mine = lane >= l0 && lane < l0 + 64 / F;
        const uint32_t c0 = mine ? (uint32_t)__builtin_popcount(kw0) : 0u;
        const uint32_t c1 = mine ? (uint32_t)__builtin_popcount(kw1) : 0u;
        const uint32_t incl = wave_incl_scan_u32(c0 + c1);
        uint32_t o = incl - c0 - c1;
        int32_t p0 = kp0, p1 = kp1;
        for (uint32_t m = mine ? kw0 : 0u; m; m &= m - 1) ents[o++] = (uint32_t)(s0 + __builtin_ctz(m)) | ((uint32_t)p0++ << 16);
        for (uint32_t m = mine ? kw1 : 0u; m; m &= m - 1)
            ents[o++] = (uint32_t)(s0 + __builtin_ctz(m)) | (1u << 15) | ((uint32_t)p1++ << 16);
        if (lane == 63) *nent_sh = (int32_t)incl;
    }
    __syncthreads();
    const int32_t nent = *nent_sh;
    for (int32_t i0 = 0; i0 < nent; i0 += OR_CH) {
        const int cnt = nent - i0 < OR_CH ? nent - i0 : OR_CH;  // entries this round
        for (int q = tid; q < cnt * nvec; q += ONE_NT) {
            const int i = q / nvec, c = q - i * nvec;
            const int32_t slot = (int32_t)(ents[i0 + i] & 0x7fffu);
            const int64_t j = a.cand ? (int64_t)a.cand[(int64_t)bq * a.n + slot] : (int64_t)slot;
            rs_stage_piece<F32>(a.kI, a.kfp4, (size_t)b * a.N + j, a.dI, c, &krow[i][c * EPV]);
        }
        __syncthreads();
        const int ew = wave * RS_EPW;
        if (ew < cnt) {
            double sc = rs_wave_scores<F32, 4>(a.qI, a.w, bq, a.HI, a.dI, qsh, krow, ew, tl[wave]);
            if (a.bf16key) sc = bf16_round_key(sc);
            if (lane < RS_EPW && ew + lane < cnt) {
                const uint32_t e = ents[i0 + ew + lane];
                a.band_score[((e >> 15) & 1u ? row1 : row0) + (e >> 16)] = sc;
            }
        }
        __syncthreads();  // the staged rows are replaced next round
    }
}

// Smallest key in [lk, hk] whose bin is >= target (hk + 1 if none): a 64-way
// search in a window of +-2048 keys around the estimate lo + target / inv,
// checked to bracket the answer, else over the whole range.
__device__ uint32_t edge_key(uint32_t lk, uint32_t hk, int target, float lo, float inv) {
    if (inv > 0.f) {
        const uint32_t ke0 = fkey(lo + (float)target / inv);
        const uint32_t ke = ke0 < lk ? lk : (ke0 > hk ? hk : ke0);
        const uint32_t L = ke - lk > 2048u ? ke - 2048u : lk;
        const uint32_t R = hk - ke > 2048u ? ke + 2048u : hk;
        const bool okL = L == lk || sel_bin(fkey_inv(L), lo, inv) < target;
        const bool okR = R == hk || sel_bin(fkey_inv(R), lo, inv) >= target;
        if (okL && okR) return wave_search_bin(L, R, target, lo, inv);
    }
    return wave_search_bin(lk, hk, target, lo, inv);
}

template <bool CERT>
__global__ __launch_bounds__(ONE_NT) void k_sel_one(OneArgs a) {
    static_assert(NB == 2 * ONE_NT, "a thread takes two bins of the suffix scan");
    __shared__ uint32_t hist[NB + NB_SPARE];  // bins, then sel_count's spare words
    __shared__ uint32_t bm[ONE_N / 32];
    __shared__ uint32_t red[ONE_NT / 64];
    __shared__ f32x4 rred[ONE_NT / 64];
    __shared__ int bstar_sh[2];
    __shared__ double thr_sh[2];
    __shared__ int32_t band_cnt_sh[2], in_cnt_sh[2];
    // exact mode's finishing scratch
    __shared__ uint64_t key_lds[CERT ? 1 : BANDFAST];
    __shared__ int32_t slot_lds[CERT ? 1 : BANDFAST];
    __shared__ int32_t out_lds[CERT ? 1 : ONE_OUT];
    // certified band rescoring (a.qI set): chunks of the band, query rows, head terms
    __shared__ __attribute__((aligned(16))) double or_krow[CERT ? OR_CH : 1][RS_MAXD];
    __shared__ u32x4 or_q[CERT ? 64 : 1][RS_QS];
    __shared__ double or_tl[CERT ? ONE_NT / 64 : 1][RS_EPW][64];
    __shared__ uint32_t or_ents[CERT ? 2 * ONE_N / (ONE_NT / 64) : 1];  // a replica's band entries
    __shared__ int32_t or_nent;
    const int bq = blockIdx.x;
    const int rep = CERT ? (int)blockIdx.y : 0;  // replica: only replica 0 writes the selection
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int n = (int)a.n;
    const int64_t base = (int64_t)bq * a.n;
    const double sumwq = CERT ? a.sumwq[bq] : 0.0;  // in flight with the scores

    // scores (all loads in flight, slots past n read the last slot and are
    // dropped), candidate filter, tile statistics
    float v[ONE_SPT];
    const int s0 = ONE_SPT * tid;
    const float *sp = a.scores + base;
    const int32_t *cp = a.cand ? a.cand + base : nullptr;
    if (s0 + ONE_SPT <= n && ((reinterpret_cast<uintptr_t>(sp) | reinterpret_cast<uintptr_t>(cp)) & 15) == 0) {
        // whole word in range: 16-byte loads
#pragma unroll
        for (int i = 0; i < ONE_SPT; i += 4) {
            const f32x4 q4 = *reinterpret_cast<const f32x4 *>(sp + s0 + i);
            v[i] = q4[0], v[i + 1] = q4[1], v[i + 2] = q4[2], v[i + 3] = q4[3];
        }
        if (cp) {
#pragma unroll
            for (int i = 0; i < ONE_SPT; i += 4) {
                const u32x4 c4 = *reinterpret_cast<const u32x4 *>(cp + s0 + i);
#pragma unroll
                for (int e = 0; e < 4; e++)
                    if ((int32_t)c4[e] < 0) v[i + e] = NEG_INF;
            }
        }
    } else {
        // the ragged last word (slots past n read the last slot and are dropped)
#pragma unroll
        for (int i = 0; i < ONE_SPT; i++) {
            const int sl = s0 + i < n ? s0 + i : n - 1;
            v[i] = sp[sl];
            if (cp && cp[sl] < 0) v[i] = NEG_INF;
            if (s0 + i >= n) v[i] = NEG_INF;
        }
    }
    for (int i = tid; i < NB; i += ONE_NT) hist[i] = 0;
    if (tid < 2) {
        bstar_sh[tid] = -1;
        band_cnt_sh[tid] = 0;
        in_cnt_sh[tid] = 0;
    }
    float lo = POS_INF, hi = NEG_INF, km = 0.f;
    uint32_t c = 0;
    const bool have_range = a.stats != nullptr;
    if (have_range) {
        for (int t = tid; t < a.ntiles; t += ONE_NT) {
            const TileStat st = a.stats[(size_t)bq * a.ntiles + t];
            lo = fminf(lo, st.smin);
            hi = fmaxf(hi, st.smax);
            km = fmaxf(km, st.kmax2);
            c += st.nvalid;
        }
    } else {
#pragma unroll
        for (int i = 0; i < ONE_SPT; i++)
            if (v[i] != NEG_INF) {
                lo = fminf(lo, v[i]);
                hi = fmaxf(hi, v[i]);
                c++;
            }
    }
    // the band rescoring's query rows (heads 0 .. 63), in flight from here
    u32x4 rq[OR_QPT];
    const int r_nvec = a.dI * (a.rs_f32 ? 4 : 2) / 16;
    const int r_nqv = (a.HI < 64 ? a.HI : 64) * r_nvec;
    if constexpr (CERT) {
        if (a.qI) {
            const u32x4 *src = reinterpret_cast<const u32x4 *>(static_cast<const char *>(a.qI) +
                                                               (size_t)bq * a.HI * a.dI * (a.rs_f32 ? 4 : 2));
#pragma unroll
            for (int i = 0; i < OR_QPT; i++) rq[i] = src[min(tid + ONE_NT * i, r_nqv - 1)];
        }
    }
    lo = wave_min(lo);
    hi = wave_max(hi);
    km = wave_max(km);
    c = wave_sum_u32(c);
    if (lane == 0) rred[wave] = f32x4{lo, hi, km, __uint_as_float(c)};
    __syncthreads();
    uint32_t nvalid = 0;
    {
        f32x4 rv[ONE_NT / 64];
#pragma unroll
        for (int i = 0; i < ONE_NT / 64; i++) rv[i] = rred[i];
#pragma unroll
        for (int i = 0; i < ONE_NT / 64; i++) {
            lo = fminf(lo, rv[i][0]);
            hi = fmaxf(hi, rv[i][1]);
            km = fmaxf(km, rv[i][2]);
            nvalid += __float_as_uint(rv[i][3]);
        }
    }
    const float inv = (nvalid > 0 && hi - lo > 0.f) ? (float)NB / (hi - lo) : 0.f;

    // histogram from registers (a thread whose slots all lie past n has none)
    if (s0 < n) sel_count(v, lo, inv, hist);
    if constexpr (CERT) {
        if (a.qI) {
#pragma unroll
            for (int i = 0; i < OR_QPT; i++) {
                const int vq = tid + ONE_NT * i;
                if (vq < r_nqv) or_q[vq / r_nvec][vq % r_nvec] = rq[i];
            }
        }
    }
    __syncthreads();
    // Suffix counts, top bin first: thread t takes bins NB-1-2t and NB-2-2t;
    // an inclusive scan in thread order gives S = the number of scores in bins
    // >= NB-2-2t, and the thread whose pair holds the K-th largest score names
    // its bin b* for each target.
    {
        const uint32_t h_hi = hist[NB - 1 - 2 * tid], h_lo = hist[NB - 2 - 2 * tid];
        const uint32_t incl = wave_incl_scan_u32(h_hi + h_lo);
        if (lane == 63) red[wave] = incl;
        __syncthreads();
        uint32_t before = 0;
#pragma unroll
        for (int i = 0; i < ONE_NT / 64; i++) before += i < wave ? red[i] : 0u;
        const uint32_t S = before + incl;          // scores in bins >= NB-2-2t
        const uint32_t S_prev = S - h_hi - h_lo;   // scores in bins >= NB-2t
        const uint32_t c_hi = S_prev + h_hi;       // scores in bins >= NB-1-2t
        for (int tg = 0; tg < a.ntgt; tg++) {
            const uint32_t K = (uint32_t)a.K[tg];
            if (nvalid > K) {
                if (c_hi >= K && S_prev < K) bstar_sh[tg] = NB - 1 - 2 * tid;
                else if (S >= K && c_hi < K) bstar_sh[tg] = NB - 2 - 2 * tid;
            }
        }
    }
    __syncthreads();

    const int64_t nwords = (a.n + 31) / 32;
    uint32_t kw0 = 0, kw1 = 0;  // this thread's band bits and their first list positions per target
    int32_t kp0 = 0, kp1 = 0;
    for (int tg = 0; tg < a.ntgt; tg++) {
        const int K = a.K[tg];
        const int bstar = bstar_sh[tg];
        double tlo = -__builtin_inf(), thi = -__builtin_inf();
        if (bstar >= 0) {
            // [a, z] = float values >= lo whose bin is b* (bin() is monotone);
            // wave 0 finds the lower edge and its threshold, wave 1 the upper
            if (wave < 2) {
                const uint32_t lk = fkey(lo), hk = 0xff7fffffu;
                uint32_t kk = hk;
                if (wave == 0) kk = edge_key(lk, hk, bstar, lo, inv);
                else if (bstar + 1 < NB) kk = edge_key(lk, hk, bstar + 1, lo, inv) - 1;
                double E = 0.0;
                if constexpr (CERT) {
                    E = score_bound(sqrt((double)km * (1.0 + ldexp(1.0, -10))), sumwq * (1.0 + ldexp(1.0, -30)),
                                    a.HI, a.dI);
                    if (a.bf16key) E = bf16_key_bound(E, fmax(fabs((double)lo), fabs((double)hi)));
                }
                if (lane == 0) thr_sh[wave] = wave == 0 ? thr_lo(fkey_inv(kk), E) : thr_hi(fkey_inv(kk), E);
            }
            __syncthreads();
            tlo = thr_sh[0];
            thi = thr_sh[1];
        }
        // IN: x > thi  <=>  x > f_hi;  BAND: x >= tlo  <=>  x >= f_lo  (x is a float)
        const float f_hi = f32_down(thi), f_lo = f32_up(tlo);
        int32_t *band = a.band + ((size_t)tg * gridDim.x + bq) * a.band_cap;
        // bit i of word t: slot 32 t + i is IN (resp. BAND); -inf (no score)
        // is neither, since f_lo is finite
        const float f_lo2 = fmaxf(f_lo, -__FLT_MAX__);
        uint32_t win = 0, wbnd = 0;
#pragma unroll
        for (int i = 0; i < ONE_SPT; i++) {
            const float x = v[i];
            win |= (x > f_hi ? 1u : 0u) << i;
            wbnd |= (x <= f_hi && x >= f_lo2 ? 1u : 0u) << i;
        }
        bm[tid] = win;
        if constexpr (CERT) {
            // list positions and counts by one block scan of the packed word
            // counts (band in the low half, IN in the high half: each total
            // is at most 32,768): the band list in slot order, the same in
            // every replica of the query
            uint32_t tot = 0;
            const uint32_t cw = (uint32_t)__builtin_popcount(wbnd) | ((uint32_t)__builtin_popcount(win) << 16);
            const uint32_t pre = block_excl_scan_u32<ONE_NT>(cw, red, tot);
            const int32_t bpos = (int32_t)(pre & 0xffffu), ipos = (int32_t)(pre >> 16);
            const int32_t nb = (int32_t)(tot & 0xffffu), in_cnt = (int32_t)(tot >> 16);
            if (tg == 0) kw0 = wbnd, kp0 = bpos;
            else kw1 = wbnd, kp1 = bpos;
            if (rep == 0) {
                int32_t pos = bpos;
                for (uint32_t m = wbnd; m; m &= m - 1) band[pos++] = s0 + __builtin_ctz(m);
                uint32_t *gbm = a.bitmap + ((size_t)tg * gridDim.x + bq) * a.nwords;
                if (tid < nwords) gbm[tid] = win;
                if (tg == 0 && a.in_list) {
                    // the IN entries in slot order
                    int32_t *il = a.in_list + (size_t)bq * K;
                    int32_t p2 = ipos;
                    for (uint32_t m = win; m; m &= m - 1) {
                        const int sl = s0 + __builtin_ctz(m);
                        il[p2++] = cp ? cp[sl] : sl;
                    }
                }
                if (tid == 0) {
                    SelTarget t;
                    t.lo = tlo;
                    t.hi = thi;
                    t.K = K;
                    t.in_cnt = in_cnt;
                    t.band_cnt = nb;
                    t.pad = 0;
                    a.sq[bq].t[tg] = t;
                    if (tg == 0) a.sq[bq].nvalid = (int32_t)nvalid;
                }
            }
        } else {
            // band slots: one block-wide counter update per wave, then each lane
            // writes the slots of its word at its offset within the wave
            const uint32_t nbw = (uint32_t)__builtin_popcount(wbnd);
            const uint32_t incl = wave_incl_scan_u32(nbw);
            const uint32_t wtot = __builtin_amdgcn_readlane(incl, 63);
            const uint32_t nin = wave_sum_u32((uint32_t)__builtin_popcount(win));
            int32_t wbase = 0;
            if (lane == 0) {
                if (wtot) wbase = atomicAdd(&band_cnt_sh[tg], (int32_t)wtot);
                if (nin) atomicAdd(&in_cnt_sh[tg], (int32_t)nin);
            }
            wbase = __builtin_amdgcn_readlane(wbase, 0);
            {
                int32_t pos = wbase + (int32_t)(incl - nbw);
                for (uint32_t m = wbnd; m; m &= m - 1) band[pos++] = s0 + __builtin_ctz(m);
            }
            __syncthreads();
            const int32_t in_cnt = in_cnt_sh[tg];
            const int32_t nb = band_cnt_sh[tg];
            __threadfence_block();
            __syncthreads();
            int32_t *dst = (tg == 0 ? a.out0 : a.out1) + (size_t)bq * K;
            finish_target<ONE_NT>(bm, nwords, a.n, K, in_cnt, nb, band, nullptr, a.scores + base,
                                  a.cand ? a.cand + base : nullptr, dst, tg == 0 && a.count0 ? a.count0 + bq : nullptr,
                                  key_lds, slot_lds, out_lds, ONE_OUT, red);
        }
        __syncthreads();
    }
    if constexpr (CERT) {
        if (a.qI) {
            if (a.rs_f32)
                one_rescore<true>(a, bq, rep, s0, kw0, kw1, kp0, kp1, or_ents, &or_nent, or_krow, or_q, or_tl);
            else
                one_rescore<false>(a, bq, rep, s0, kw0, kw1, kp0, kp1, or_ents, &or_nent, or_krow, or_q, or_tl);
        }
    }
}

// Rows of at most RS_ROWB bytes: a block takes RS_EPB consecutive band
// entries of one query.  Its band slots are read speculatively with the target
// record; then the query rows of the first 64 heads (coalesced, staged in LDS)
// and the block's key rows (one 16-byte load per thread, staged in LDS already
// converted to binary64) are in flight together, so the dot products read the
// key values as broadcast operands and spend the double-precision unit on the
// fused multiply-adds alone.  Each wave
// runs RS_EPW entries as independent binary64 chains (lane h: head h), then
// lane e sums entry e's head terms in order.  Two entries per wave spread a
// query's band over about as many waves as the chip has SIMDs.  Blocks loop
// over the list when it is longer than the grid.
template <bool F32>
__global__ __launch_bounds__(RS_NT, 2) void k_sel_rescore(RescoreKArgs a) {
#pragma clang fp contract(off)
    constexpr int QPT = 64 * (RS_ROWB / 16) / RS_NT;
    __shared__ __attribute__((aligned(16))) double krow_lds[RS_EPB][RS_MAXD];
    __shared__ u32x4 qsh[64][RS_QS];
    __shared__ double tl[RS_NT / 64][RS_EPW][64];
    constexpr int ESZ = F32 ? 4 : 2;
    constexpr int EPV = 16 / ESZ;  // elements per 16-byte vector
    const int bq = blockIdx.y;
    const int b = bq / a.Q;
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int nvec = a.dI * ESZ / 16;  // 16-byte vectors per row
    const size_t row0 = (size_t)bq * a.band_cap, row1 = ((size_t)gridDim.y + bq) * a.band_cap;
    // speculative: this block's first entries as target-0 slots
    const int32_t eb0 = blockIdx.x * RS_EPB;
    const int32_t my_e = eb0 + tid / nvec;  // entry whose row chunk this thread stages
    const int32_t spec = (tid < RS_EPB * nvec && my_e < a.band_cap) ? a.band[row0 + my_e] : 0;
    const SelQuery sqv = a.sq[bq];
    const int32_t nb0 = sqv.t[0].band_cnt, nb1 = a.ntgt > 1 ? sqv.t[1].band_cnt : 0;
    const int32_t total = nb0 + nb1;
    if (eb0 >= total) return;
    // query rows of heads 0 .. min(HI, 64) - 1, row-major in 16-byte vectors
    const int nqv = (a.HI < 64 ? a.HI : 64) * nvec;
    u32x4 qst[QPT];
    {
        const u32x4 *qsrc = reinterpret_cast<const u32x4 *>(static_cast<const char *>(a.qI) + (size_t)bq * a.HI * a.dI * ESZ);
#pragma unroll
        for (int i = 0; i < QPT; i++)
            if (tid + RS_NT * i < nqv) qst[i] = qsrc[tid + RS_NT * i];
    }
    bool q_staged = false;
    for (int32_t e0 = eb0; e0 < total; e0 += gridDim.x * RS_EPB) {
        // stage the key rows of entries e0 .. e0 + RS_EPB - 1 as binary64
        for (int q = tid; q < RS_EPB * nvec; q += RS_NT) {
            const int i = q / nvec, c = q - i * nvec;
            const int32_t e = e0 + i;
            if (e < total) {
                const int32_t slot = (e0 == eb0 && q == tid && e < nb0)
                                         ? spec
                                         : (e < nb0 ? a.band[row0 + e] : a.band[row1 + (e - nb0)]);
                const int64_t j = a.cand ? (int64_t)a.cand[(int64_t)bq * a.n + slot] : (int64_t)slot;
                rs_stage_piece<F32>(a.kI, a.kfp4, (size_t)b * a.N + j, a.dI, c, &krow_lds[i][c * EPV]);
            }
        }
        if (!q_staged) {
#pragma unroll
            for (int i = 0; i < QPT; i++) {
                const int v = tid + RS_NT * i;
                if (v < nqv) qsh[v / nvec][v % nvec] = qst[i];
            }
            q_staged = true;
        }
        __syncthreads();
        const int ew = wave * RS_EPW;  // this wave's first entry in the block
        double sc = rs_wave_scores<F32>(a.qI, a.w, bq, a.HI, a.dI, qsh, krow_lds, ew, tl[wave]);
        const int32_t e = e0 + ew + lane;
        if (a.bf16key) sc = bf16_round_key(sc);
        if (lane < RS_EPW && e < total) {
            if (e < nb0) a.band_score[row0 + e] = sc;
            else a.band_score[row1 + (e - nb0)] = sc;
        }
        __syncthreads();  // the staged rows are replaced next round
    }
}

// Rows longer than RS_ROWB: one wave per band entry.  The entry's slot is read
// speculatively with the target record, and the wave's query rows and head
// weights before the first entry.
template <bool F32>
__global__ __launch_bounds__(RS_NT) void k_sel_rescore_wide(RescoreKArgs a) {
#pragma clang fp contract(off)
    __shared__ double tl[RS_NT / 64][64];
    constexpr int ESZ = F32 ? 4 : 2;
    const int bq = blockIdx.y;
    const int b = bq / a.Q;
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    constexpr int NW = RS_NT / 64;
    const int nvec = a.dI * ESZ / 16;  // 16-byte vectors per row (a whole number, checked on the host)
    const int32_t e0 = blockIdx.x * NW + wave;
    // speculative: the first entry's slot in each target list
    const size_t row0 = (size_t)bq * a.band_cap, row1 = ((size_t)gridDim.y + bq) * a.band_cap;
    const int32_t spec0 = e0 < a.band_cap ? a.band[row0 + e0] : 0;
    const SelQuery sqv = a.sq[bq];
    const int32_t nb0 = sqv.t[0].band_cnt, nb1 = a.ntgt > 1 ? sqv.t[1].band_cnt : 0;
    const int32_t total = nb0 + nb1;
    if (e0 >= total) return;
    for (int h0 = 0; h0 < a.HI; h0 += 64) {
        const int h = h0 + lane;
        const int hc = h < a.HI ? h : a.HI - 1;  // idle lanes recompute the last head, unused
        const u32x4 *qrow = reinterpret_cast<const u32x4 *>(static_cast<const char *>(a.qI) +
                                                            ((size_t)bq * a.HI + hc) * a.dI * ESZ);
        const double wh = (double)a.w[(size_t)bq * a.HI + hc];
        u32x4 qv[RS_VB];
        const bool qcached = nvec <= RS_VB;  // the query row stays in registers across entries
        if (qcached) {
#pragma unroll
            for (int u = 0; u < RS_VB; u++)
                if (u < nvec) qv[u] = qrow[u];
        }
        for (int32_t e = e0; e < total; e += gridDim.x * NW) {
            const int tg = e < nb0 ? 0 : 1;
            const int32_t pos = tg == 0 ? e : e - nb0;
            const int32_t slot = (e == e0 && tg == 0) ? spec0 : a.band[(tg == 0 ? row0 : row1) + pos];
            const int64_t j = a.cand ? (int64_t)a.cand[(int64_t)bq * a.n + slot] : (int64_t)slot;
            const u32x4 *krow = reinterpret_cast<const u32x4 *>(static_cast<const char *>(a.kI) +
                                                                ((size_t)b * a.N + j) * a.dI * ESZ);
            double dot = 0.0;
            for (int v0 = 0; v0 < nvec; v0 += RS_VB) {
                u32x4 kv[RS_VB];
#pragma unroll
                for (int u = 0; u < RS_VB; u++)
                    if (v0 + u < nvec) {
                        if (!qcached) qv[u] = qrow[v0 + u];
                        kv[u] = krow[v0 + u];
                    }
#pragma unroll
                for (int u = 0; u < RS_VB; u++)
                    if (v0 + u < nvec) dot = dot_vec<F32>(dot, qv[u], kv[u]);
            }
            const double rl = dot > 0.0 ? dot : 0.0;
            tl[wave][lane] = wh * rl;
            __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
            __builtin_amdgcn_wave_barrier();
            __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
            if (lane == 0) {
                // head terms t_h0, t_h0+1, ... added in order (read 16 at a time)
                const int hn = a.HI - h0 < 64 ? a.HI - h0 : 64;
                double sc = h0 == 0 ? 0.0 : a.band_score[(tg == 0 ? row0 : row1) + pos];
                for (int c0 = 0; c0 < hn; c0 += 16) {
                    double tv[16];
#pragma unroll
                    for (int i = 0; i < 16; i++) tv[i] = tl[wave][c0 + i];
#pragma unroll
                    for (int i = 0; i < 16; i++)
                        if (c0 + i < hn) sc = sc + tv[i];
                }
                if (a.bf16key && h0 + 64 >= a.HI) sc = bf16_round_key(sc);  // the last head pass
                a.band_score[(tg == 0 ? row0 : row1) + pos] = sc;
            }
            __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
            __builtin_amdgcn_wave_barrier();
            __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
        }
    }
}

// ------------------------------------------------------- one-block finish
// Certified finish of the one-block path: the IN bitmap (one word per
// thread), the target record and the first ONE_NT band entries with their
// binary64 scores arrive in one round of loads.  Each band entry is ranked by
// counting the entries ahead of it in (score descending, slot ascending)
// order; the best K - |IN| join the bitmap, which is compacted in slot order
// through LDS.  Larger bands or outputs take the general path.
struct BandEnt {
    uint64_t key;
    int32_t slot, pad;
};

__global__ __launch_bounds__(ONE_NT) void k_sel_finish_one(const float *__restrict__ scores,
                                                           const int32_t *__restrict__ cand, int64_t n, int ntgt,
                                                           const SelQuery *__restrict__ sq, const uint32_t *bitmap,
                                                           int64_t nwords, const int32_t *band, const double *band_score,
                                                           int64_t band_cap, int32_t *out0, int32_t *count0,
                                                           int32_t *out1, int tg0) {
    __shared__ uint32_t bm[ONE_N / 32];
    __shared__ __attribute__((aligned(16))) BandEnt ent[ONE_NT];
    __shared__ int32_t out_lds[ONE_OUT];
    __shared__ uint32_t red[ONE_NT / 64];
    const int bq = blockIdx.x, tid = threadIdx.x;
    for (int tg = tg0; tg < ntgt; tg++) {
        const size_t row = (size_t)tg * gridDim.x + bq;
        const SelTarget t = sq[bq].t[tg];
        const uint32_t wv = tid < nwords ? bitmap[row * nwords + tid] : 0u;
        const int32_t bsl = tid < band_cap ? band[row * band_cap + tid] : 0;
        const double bsc = tid < band_cap ? band_score[row * band_cap + tid] : 0.0;
        int32_t *dst = (tg == 0 ? out0 : out1) + (size_t)bq * t.K;
        int32_t *cdst = tg == 0 && count0 ? count0 + bq : nullptr;
        const int32_t nb = t.band_cnt, r = t.K - t.in_cnt;
        bm[tid] = wv;
        if (nb > ONE_NT || t.K > ONE_OUT) {  // general path
            __syncthreads();
            finish_target<ONE_NT>(bm, nwords, n, t.K, t.in_cnt, nb, band + row * band_cap,
                                  band_score + row * band_cap, scores + (int64_t)bq * n,
                                  cand ? cand + (int64_t)bq * n : nullptr, dst, cdst,
                                  reinterpret_cast<uint64_t *>(out_lds), reinterpret_cast<int32_t *>(ent), out_lds,
                                  0, red);
            __syncthreads();
            continue;
        }
        if (tid < nb) {
            BandEnt be;
            be.key = dkey(bsc);
            be.slot = bsl;
            be.pad = 0;
            ent[tid] = be;
        }
        __syncthreads();
        // entry i's rank is counted by P consecutive lanes over every P-th entry
        // (all 16 waves busy, short dependent chains), then summed by a butterfly
        const int P = nb <= 128 ? 8 : nb <= 256 ? 4 : nb <= 512 ? 2 : 1;
        const int ei = tid / P, ep = tid - ei * P;
        int32_t rank = 0;
        const bool ranks = r > 0 && ei < nb;
        uint64_t ki = 0;
        int32_t si = 0;
        if (ranks) {
            ki = ent[ei].key;
            si = ent[ei].slot;
            // eight reads in flight per step
            for (int32_t j0 = ep; j0 < nb; j0 += 8 * P) {
                BandEnt bj[8];
#pragma unroll
                for (int u = 0; u < 8; u++) {
                    const int32_t j = j0 + u * P;
                    bj[u] = ent[j < nb ? j : ei];  // past the end: compare with itself (counts 0)
                }
#pragma unroll
                for (int u = 0; u < 8; u++)
                    rank += (int)((bj[u].key > ki) | ((bj[u].key == ki) & (bj[u].slot < si)));
            }
        }
        for (int o = 1; o < P; o <<= 1) rank += __shfl_xor(rank, o);
        if (ranks && ep == 0 && rank < r) atomicOr(&bm[si >> 5], 1u << (si & 31));
        __syncthreads();
        // compaction: thread tid owns bitmap word tid
        uint32_t bits = bm[tid];
        uint32_t tot;
        uint32_t pos = block_excl_scan<ONE_NT>((uint32_t)__builtin_popcount(bits), red, tot);
        while (bits) {
            const int i = __builtin_ctz(bits);
            bits &= bits - 1;
            if (pos < (uint32_t)t.K) out_lds[pos] = tid * 32 + i;
            pos++;
        }
        const int32_t kept = (int32_t)(tot < (uint32_t)t.K ? tot : (uint32_t)t.K);
        __syncthreads();
        const int32_t *cq = cand ? cand + (int64_t)bq * n : nullptr;
        for (int32_t i = tid; i < t.K; i += ONE_NT) dst[i] = i < kept ? (cq ? cq[out_lds[i]] : out_lds[i]) : -1;
        if (cdst && tid == 0) *cdst = kept;
        __syncthreads();
    }
}

// ------------------------------------------------------------------ finish
// One block per query and target: band pick + compaction, the bitmap staged
// in LDS when it fits.
constexpr int FIN_NT = 1024;
constexpr int64_t FIN_BM = 8192;   // bitmap words kept in LDS
constexpr int FIN_OUT = 16384;     // output entries staged in LDS

struct FinishArgs {
    const float *scores;
    const int32_t *cand;
    int64_t n;
    int ntgt;
    const SelQuery *sq;
    uint32_t *bitmap;
    int64_t nwords;
    const int32_t *band;
    const double *band_score;
    int64_t band_cap;
    int32_t *out0, *count0, *out1;
    int tg0;  // first target to finish
};

__global__ __launch_bounds__(FIN_NT) void k_sel_finish(FinishArgs a) {
    __shared__ __attribute__((aligned(16))) uint32_t bm_lds[FIN_BM];
    __shared__ uint64_t key_lds[BANDFAST];
    __shared__ int32_t slot_lds[BANDFAST];
    __shared__ int32_t out_lds[FIN_OUT];
    __shared__ uint32_t red[FIN_NT / 64];
    const int bq = blockIdx.x;
    {
        const int tg = a.tg0 + blockIdx.y;  // the targets of a query are finished by separate blocks
        const SelTarget t = a.sq[bq].t[tg];
        uint32_t *gbm = a.bitmap + ((size_t)tg * gridDim.x + bq) * a.nwords;
        const int32_t *list = a.band + ((size_t)tg * gridDim.x + bq) * a.band_cap;
        const double *bs = a.band_score ? a.band_score + ((size_t)tg * gridDim.x + bq) * a.band_cap : nullptr;
        int32_t *dst = (tg == 0 ? a.out0 : a.out1) + (size_t)bq * t.K;
        int32_t *cdst = tg == 0 && a.count0 ? a.count0 + bq : nullptr;
        const float *sq_scores = a.scores + (int64_t)bq * a.n;
        const int32_t *cq = a.cand ? a.cand + (int64_t)bq * a.n : nullptr;
        uint32_t *bm = gbm;
        if (a.nwords <= FIN_BM) {
            bm = bm_lds;
            if ((a.nwords & 3) == 0) {
                const int64_t nv = a.nwords / 4;
                for (int64_t v0 = threadIdx.x; v0 < nv; v0 += 4 * FIN_NT) {
                    u32x4 tmp[4];
#pragma unroll
                    for (int u = 0; u < 4; u++)
                        if (v0 + u * FIN_NT < nv) tmp[u] = reinterpret_cast<const u32x4 *>(gbm)[v0 + u * FIN_NT];
#pragma unroll
                    for (int u = 0; u < 4; u++)
                        if (v0 + u * FIN_NT < nv) reinterpret_cast<u32x4 *>(bm_lds)[v0 + u * FIN_NT] = tmp[u];
                }
            } else {
                for (int64_t wd = threadIdx.x; wd < a.nwords; wd += FIN_NT) bm_lds[wd] = gbm[wd];
            }
            __syncthreads();
        }
        finish_target<FIN_NT>(bm, a.nwords, a.n, t.K, t.in_cnt, t.band_cnt, list, bs, sq_scores, cq, dst, cdst,
                              key_lds, slot_lds, out_lds, FIN_OUT, red, false, bm == gbm);
    }
}

}  // namespace

// ------------------------------------------------------------------ host

bool rescore_supported(int dt, int dI) {
    if (dt == CSA2_FP4) return dI % 64 == 0 && dI * 2 <= RS_ROWB;  // staged kernel only
    return dI >= 1 && (dI * (dt == CSA2_F32 ? 4 : 2)) % 16 == 0;
}

SelPlan sel_plan(int BQ, int64_t n, int K0, int K1, bool certified) {
    SelPlan p;
    p.BQ = BQ;
    p.n = n;
    p.K0 = K0;
    p.K1 = K1;
    p.ntgt = K1 > 0 ? 2 : 1;
    p.ntiles = (int)((n + TILE - 1) / TILE);
    p.nchunks = (int)((n + CH - 1) / CH);
    p.nwords = (n + 31) / 32;
    p.band_cap = n;
    p.certified = certified;
    return p;
}

static bool small_path(const SelPlan &p) { return p.n <= ONE_N; }

bool sel_handoff_supported(const SelPlan &p) { return p.certified && small_path(p); }

size_t sel_workspace(const SelPlan &p, bool own_stats) {
    Carve c(nullptr, 0);
    if (own_stats && !small_path(p)) c.take<TileStat>((size_t)p.BQ * p.ntiles);
    c.take<uint32_t>((size_t)p.BQ * NB);
    c.take<SelQuery>((size_t)p.BQ);
    c.take<double>((size_t)p.BQ);  // error bounds
    c.take<uint32_t>((size_t)p.ntgt * p.BQ * p.nwords);
    c.take<int32_t>((size_t)p.ntgt * p.BQ * p.band_cap);
    if (p.certified) c.take<double>((size_t)p.ntgt * p.BQ * p.band_cap);
    if (sel_handoff_supported(p)) c.take<int32_t>((size_t)p.BQ * p.K0);  // IN list of the top-k target
    return c.used;
}



// Replicas of each query's one-block selection that share its band
// rescoring (0: the rescoring kernel does it): one per wave of the block
// (replica r takes wave r's words), or per half or quarter of a wave's lanes
// with at most 8 or 4 queries, with at most 16 queries, rows the staged
// rescoring takes (at most RS_ROWB bytes), certified selection.
static int one_rescore_replicas(const SelPlan &p, const RescoreArgs *rs) {
    if (!p.certified || !rs || !small_path(p)) return 0;
    const int rowb = rs->dI * (rs->dt == CSA2_F32 ? 4 : 2);
    if (rowb > RS_ROWB) return 0;
    if (p.BQ > 16) return 0;
    // one replica per wave's slots, or per half or quarter of a wave's lanes
    // when there are few queries, so that the grid still fills the chip
    const int f = p.BQ <= 4 ? 4 : (p.BQ <= 8 ? 2 : 1);
    return f * (ONE_NT / 64);
}

void sel_run(const SelPlan &p, const float *scores, const int32_t *cand, const TileStat *stats_in,
             const RescoreArgs *rs, int32_t *out0, int32_t *count0, int32_t *out1, void *ws, size_t ws_bytes,
             hipStream_t s, SelHandoff *handoff) {
    Carve c(ws, ws_bytes);
    TileStat *stats = const_cast<TileStat *>(stats_in);
    if (!stats && !small_path(p)) stats = c.take<TileStat>((size_t)p.BQ * p.ntiles);
    uint32_t *qhist = c.take<uint32_t>((size_t)p.BQ * NB);
    SelQuery *sq = c.take<SelQuery>((size_t)p.BQ);
    double *ebuf = c.take<double>((size_t)p.BQ);
    uint32_t *bitmap = c.take<uint32_t>((size_t)p.ntgt * p.BQ * p.nwords);
    int32_t *band = c.take<int32_t>((size_t)p.ntgt * p.BQ * p.band_cap);
    double *band_score = p.certified ? c.take<double>((size_t)p.ntgt * p.BQ * p.band_cap) : nullptr;
    int32_t *in_list = sel_handoff_supported(p) ? c.take<int32_t>((size_t)p.BQ * p.K0) : nullptr;
    if (c.used > ws_bytes) throw Error(CSA2_EWORKSPACE, "selection workspace too small");
    if (handoff && !sel_handoff_supported(p)) throw Error(CSA2_EINTERNAL, "selection hand-off not supported");
    if (p.certified && (!rs || !rs->sumwq)) throw Error(CSA2_EINTERNAL, "certified selection needs query norms");

    if (small_path(p)) {
        OneArgs a{};
        a.scores = scores;
        a.cand = cand;
        a.n = p.n;
        a.K[0] = p.K0;
        a.K[1] = p.K1;
        a.ntgt = p.ntgt;
        a.stats = stats;
        a.ntiles = p.ntiles;
        if (rs) {
            a.sumwq = rs->sumwq;
            a.HI = rs->HI;
            a.dI = rs->dI;
        }
        a.out0 = out0;
        a.count0 = count0;
        a.out1 = out1;
        a.sq = sq;
        a.bitmap = bitmap;
        a.nwords = p.nwords;
        a.band = band;
        a.band_cap = p.band_cap;
        a.in_list = handoff ? in_list : nullptr;
        a.bf16key = p.certified && p.bf16key ? 1 : 0;
        // few queries: the band's binary64 rescoring joins this kernel, split
        // over replicas of each query's block that repeat its selection (the
        // chip has CUs to spare; one launch and one kernel boundary fewer)
        const int reps = one_rescore_replicas(p, rs);
        if (reps) {
            a.qI = rs->qI;
            a.rs_f32 = rs->dt == CSA2_F32 ? 1 : 0;
            a.kfp4 = rs->dt == CSA2_FP4 ? 1 : 0;
            a.w = rs->w;
            a.kI = rs->kI;
            a.Q = rs->Q;
            a.N = rs->N;
            a.band_score = band_score;
        }
        if (p.certified) hipLaunchKernelGGL(k_sel_one<true>, dim3(p.BQ, reps ? reps : 1), dim3(ONE_NT), 0, s, a);
        else hipLaunchKernelGGL(k_sel_one<false>, dim3(p.BQ), dim3(ONE_NT), 0, s, a);
        check_launch("selection (one block per query)");
        if (!p.certified) return;
    } else {
        if (!stats_in) {
            hipLaunchKernelGGL(k_sel_stats, dim3(p.ntiles, p.BQ), dim3(256), 0, s, scores, cand, p.n, p.ntiles,
                               stats);
            check_launch("selection stats");
        }
        hipLaunchKernelGGL(k_sel_range, dim3(p.BQ), dim3(256), 0, s, stats, p.ntiles, sq, qhist,
                           p.certified ? rs->sumwq : nullptr, p.certified ? rs->HI : 0, p.certified ? rs->dI : 0,
                           p.certified ? ebuf : nullptr, p.certified && p.bf16key ? 1 : 0);
        check_launch("selection range");
        // few queries: smaller blocks of work, so that the grid still fills the chip
        const bool few = (int64_t)p.BQ * ((p.nchunks + HIST_CPB - 1) / HIST_CPB) < 256;
        if (few)
            hipLaunchKernelGGL(k_sel_hist<1>, dim3(p.nchunks, p.BQ), dim3(256), 0, s, scores, cand, p.n, sq, qhist);
        else
            hipLaunchKernelGGL(k_sel_hist<HIST_CPB>, dim3((p.nchunks + HIST_CPB - 1) / HIST_CPB, p.BQ), dim3(256), 0,
                               s, scores, cand, p.n, sq, qhist);
        check_launch("selection histogram");
        hipLaunchKernelGGL(k_sel_find, dim3(p.BQ), dim3(256), 0, s, qhist, p.K0, p.K1, p.certified ? ebuf : nullptr, sq);
        check_launch("selection find");
        const int nblk4 = (int)((p.nwords + 256 * CLS_WPT_MAX - 1) / (256 * CLS_WPT_MAX));
        if ((int64_t)p.BQ * nblk4 < 256)
            hipLaunchKernelGGL(k_sel_classify<1>, dim3((unsigned)((p.nwords + 255) / 256), p.BQ), dim3(256), 0, s,
                               scores, cand, p.n, p.ntgt, sq, bitmap, p.nwords, band, p.band_cap);
        else
            hipLaunchKernelGGL(k_sel_classify<CLS_WPT_MAX>, dim3(nblk4, p.BQ), dim3(256), 0, s, scores, cand, p.n,
                               p.ntgt, sq, bitmap, p.nwords, band, p.band_cap);
        check_launch("selection classify");
    }
    if (p.certified && !(small_path(p) && one_rescore_replicas(p, rs))) {
        RescoreKArgs r{};
        r.qI = rs->qI;
        r.dt = rs->dt;
        r.kfp4 = rs->dt == CSA2_FP4;
        r.w = rs->w;
        r.kI = rs->kI;
        r.Q = rs->Q;
        r.HI = rs->HI;
        r.dI = rs->dI;
        r.N = rs->N;
        r.cand = cand;
        r.n = p.n;
        r.ntgt = p.ntgt;
        r.sq = sq;
        r.band = band;
        r.band_score = band_score;
        r.band_cap = p.band_cap;
        r.bf16key = p.bf16key ? 1 : 0;
        const int rowb = rs->dI * (rs->dt == CSA2_F32 ? 4 : 2);
        if (rowb <= RS_ROWB) {
            // about 256 entries per query per round at 32,768 slots, more for longer
            // rows of scores (the band grows with the density of scores); the grid
            // stays resident at once (two blocks per CU: longer bands loop over
            // rounds instead of queueing blocks), and idle blocks exit at once
            int64_t want = (int64_t)256 * ((p.n + ONE_N - 1) / ONE_N);
            int nblk = (int)((want < 1024 ? want : 1024) / RS_EPB);
            if ((int64_t)nblk * p.BQ > 512) nblk = (int)(512 / p.BQ) > 1 ? (int)(512 / p.BQ) : 1;
            if (rs->dt == CSA2_F32) hipLaunchKernelGGL(k_sel_rescore<true>, dim3(nblk, p.BQ), dim3(RS_NT), 0, s, r);
            else hipLaunchKernelGGL(k_sel_rescore<false>, dim3(nblk, p.BQ), dim3(RS_NT), 0, s, r);
        } else {
            int nblk = 4096 / p.BQ / (RS_NT / 64);
            nblk = nblk < 2 ? 2 : (nblk > 64 ? 64 : nblk);
            if (rs->dt == CSA2_F32) hipLaunchKernelGGL(k_sel_rescore_wide<true>, dim3(nblk, p.BQ), dim3(RS_NT), 0, s, r);
            else hipLaunchKernelGGL(k_sel_rescore_wide<false>, dim3(nblk, p.BQ), dim3(RS_NT), 0, s, r);
        }
        check_launch("selection rescore");
    }
    int tg0 = 0;
    if (handoff) {
        *handoff = SelHandoff{sq, in_list, p.K0, bitmap, p.nwords, band, band_score, p.band_cap, cand, p.n, out0, count0};
        if (p.ntgt == 1) return;
        tg0 = 1;  // the pool is finished here
    }
    if (small_path(p)) {
        hipLaunchKernelGGL(k_sel_finish_one, dim3(p.BQ), dim3(ONE_NT), 0, s, scores, cand, p.n, p.ntgt, sq, bitmap,
                           p.nwords, band, band_score, p.band_cap, out0, count0, out1, tg0);
        check_launch("selection finish");
        return;
    }
    FinishArgs f{};
    f.scores = scores;
    f.cand = cand;
    f.n = p.n;
    f.ntgt = p.ntgt;
    f.sq = sq;
    f.bitmap = bitmap;
    f.nwords = p.nwords;
    f.band = band;
    f.band_score = band_score;
    f.band_cap = p.band_cap;
    f.out0 = out0;
    f.count0 = count0;
    f.out1 = out1;
    f.tg0 = tg0;
    hipLaunchKernelGGL(k_sel_finish, dim3(p.BQ, p.ntgt - tg0), dim3(FIN_NT), 0, s, f);
    check_launch("selection finish");
}

}  // namespace csa2
