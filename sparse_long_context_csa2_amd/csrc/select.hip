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
//              sequential operation order of the definition (one wave per
//              entry; the products of bf16/fp32 inputs are exact in binary64,
//              so a fused multiply-add equals the rounded product + add).
//  5 band+compact: rank the BAND entries by (exact score, slot) and keep the
//              first K - |IN|; then compact the bitmap in slot order into the
//              ascending index list.
#include "internal.h"

namespace csa2 {

constexpr int NB = 2048;        // histogram bins
constexpr int CH = 8192;        // slots per chunk (256 threads x 32)
constexpr int BANDFAST = 2048;  // largest band ranked by pairwise counting

struct SelTarget {
    double lo, hi;     // BAND = [lo, hi], IN = (hi, +inf)
    int32_t K;         // entries to keep
    int32_t in_cnt;    // |IN|
    int32_t band_cnt;  // |BAND|
    int32_t pad;
};
struct SelQuery {
    float lo, inv;   // bin() parameters
    int32_t nvalid;  // finite scores
    int32_t pad;
    SelTarget t[2];  // [0] = top-k, [1] = pool
};

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

// ---------------------------------------------------------------- 1: hist
__global__ __launch_bounds__(256) void k_sel_hist(const float *__restrict__ scores, const int32_t *__restrict__ cand,
                                                  int64_t n, const TileStat *__restrict__ stats, int ntiles,
                                                  int nchunks, uint32_t *__restrict__ part, SelQuery *__restrict__ sq) {
    __shared__ uint32_t hist[NB];
    __shared__ float r_min[256], r_max[256];
    __shared__ uint32_t r_n[256];
    const int bq = blockIdx.y, chunk = blockIdx.x;
    // range of the query's finite scores (fixed reduction order)
    float mn = POS_INF, mx = NEG_INF;
    uint32_t cnt = 0;
    for (int t = threadIdx.x; t < ntiles; t += 256) {
        TileStat s = stats[(size_t)bq * ntiles + t];
        mn = fminf(mn, s.smin);
        mx = fmaxf(mx, s.smax);
        cnt += s.nvalid;
    }
    r_min[threadIdx.x] = mn;
    r_max[threadIdx.x] = mx;
    r_n[threadIdx.x] = cnt;
    for (int i = threadIdx.x; i < NB; i += 256) hist[i] = 0;
    __syncthreads();
    for (int o = 128; o > 0; o >>= 1) {
        if (threadIdx.x < o) {
            r_min[threadIdx.x] = fminf(r_min[threadIdx.x], r_min[threadIdx.x + o]);
            r_max[threadIdx.x] = fmaxf(r_max[threadIdx.x], r_max[threadIdx.x + o]);
            r_n[threadIdx.x] += r_n[threadIdx.x + o];
        }
        __syncthreads();
    }
    const float lo = r_min[0], hi = r_max[0];
    const float span = hi - lo;
    const float inv = (r_n[0] > 0 && span > 0.f) ? (float)NB / span : 0.f;
    if (chunk == 0 && threadIdx.x == 0) {
        sq[bq].lo = lo;
        sq[bq].inv = inv;
        sq[bq].nvalid = (int32_t)r_n[0];
    }
    const int64_t base = (int64_t)bq * n;
    const int64_t s0 = (int64_t)chunk * CH + threadIdx.x * 32;
    for (int i = 0; i < 32; i++) {
        float v;
        if (slot_score(scores, cand, base, s0 + i, n, v)) atomicAdd(&hist[sel_bin(v, lo, inv)], 1u);
    }
    __syncthreads();
    uint32_t *dst = part + ((size_t)bq * nchunks + chunk) * NB;
    for (int i = threadIdx.x; i < NB; i += 256) dst[i] = hist[i];
}

__device__ __forceinline__ double thr_lo(float a, double E) {
    if (E > 0.0) return (double)a - 2.0 * E * (1.0 + ldexp(1.0, -20)) - fabs((double)a) * ldexp(1.0, -50);
    return (double)a;
}
__device__ __forceinline__ double thr_hi(float z, double E) {
    if (E > 0.0) return (double)z + 2.0 * E * (1.0 + ldexp(1.0, -20)) + fabs((double)z) * ldexp(1.0, -50);
    return (double)z;
}

// ---------------------------------------------------------------- 2: find
__global__ __launch_bounds__(256) void k_sel_find(const uint32_t *__restrict__ part, int nchunks, int K0, int K1,
                                                  const double *__restrict__ ebound, SelQuery *__restrict__ sq) {
    __shared__ uint32_t cum[NB + 1];
    __shared__ int bstar;
    const int bq = blockIdx.x;
    // per-thread 8 consecutive bins, summed over chunks
    uint32_t h[8];
    uint32_t local = 0;
    for (int i = 0; i < 8; i++) {
        uint32_t acc = 0;
        int b = threadIdx.x * 8 + i;
        for (int c = 0; c < nchunks; c++) acc += part[((size_t)bq * nchunks + c) * NB + b];
        h[i] = acc;
        local += acc;
    }
    // suffix sums: cum[b] = number of finite scores in bins >= b
    __shared__ uint32_t tot[256];
    tot[threadIdx.x] = local;
    __syncthreads();
    uint32_t run = 0;
    for (int t = threadIdx.x + 1; t < 256; t++) run += tot[t];
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
                // [a, z] = the float values >= lo whose bin is b* (bisection on the
                // order-preserving key; bin() is monotone)
                const uint32_t lo_k = fkey(q.lo);
                const uint32_t hi_k = 0xff7fffffu;  // key of the largest finite float
                // a: smallest key with bin >= b*
                uint32_t L = lo_k, R = hi_k;
                while (L < R) {
                    uint32_t M = L + (R - L) / 2;
                    if (sel_bin(fkey_inv(M), q.lo, q.inv) >= bstar) R = M;
                    else L = M + 1;
                }
                const float a = fkey_inv(L);
                // z: largest key with bin <= b*
                L = lo_k;
                R = hi_k;
                while (L < R) {
                    uint32_t M = L + (R - L + 1) / 2;
                    if (sel_bin(fkey_inv(M), q.lo, q.inv) <= bstar) L = M;
                    else R = M - 1;
                }
                const float z = fkey_inv(L);
                t.lo = thr_lo(a, E);
                t.hi = thr_hi(z, E);
            }
            sq[bq].t[tgt] = t;
        }
        __syncthreads();
    }
}

// ------------------------------------------------------------ 3: classify
__global__ __launch_bounds__(256) void k_sel_classify(const float *__restrict__ scores,
                                                      const int32_t *__restrict__ cand, int64_t n, int ntgt,
                                                      SelQuery *__restrict__ sq, uint32_t *__restrict__ bitmap,
                                                      int64_t nwords, int32_t *__restrict__ band, int64_t band_cap) {
    __shared__ uint32_t buf[8];
    __shared__ uint32_t base_sh;
    const int bq = blockIdx.y;
    const int64_t word = (int64_t)blockIdx.x * 256 + threadIdx.x;
    const int64_t base = (int64_t)bq * n;
    float v[32];
    uint32_t okmask = 0;
    for (int i = 0; i < 32; i++) {
        float x = 0.f;
        if (slot_score(scores, cand, base, word * 32 + i, n, x)) okmask |= 1u << i;
        v[i] = x;
    }
    for (int tgt = 0; tgt < ntgt; tgt++) {
        const SelTarget t = sq[bq].t[tgt];
        uint32_t in = 0, bandm = 0;
        for (int i = 0; i < 32; i++) {
            if (!((okmask >> i) & 1u)) continue;
            double x = (double)v[i];
            if (x > t.hi) in |= 1u << i;
            else if (x >= t.lo) bandm |= 1u << i;
        }
        if (word < nwords) bitmap[((size_t)tgt * gridDim.y + bq) * nwords + word] = in;
        uint32_t nin = block_sum_u32<256>((uint32_t)__builtin_popcount(in), buf);
        if (threadIdx.x == 0 && nin) atomicAdd(&sq[bq].t[tgt].in_cnt, (int32_t)nin);
        uint32_t nb = (uint32_t)__builtin_popcount(bandm), tot;
        uint32_t off = block_excl_scan<256>(nb, buf, tot);
        if (threadIdx.x == 0) base_sh = tot ? (uint32_t)atomicAdd(&sq[bq].t[tgt].band_cnt, (int32_t)tot) : 0u;
        __syncthreads();
        int32_t *dst = band + ((size_t)tgt * gridDim.y + bq) * band_cap;
        uint32_t pos = base_sh + off;
        while (bandm) {
            int i = __builtin_ctz(bandm);
            bandm &= bandm - 1;
            dst[pos++] = (int32_t)(word * 32 + i);
        }
        __syncthreads();
    }
}

// ------------------------------------------------- shared finishing steps

__device__ __forceinline__ uint32_t load_word(const uint32_t *p) {
    return __hip_atomic_load(p, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

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


// Pick the best r = K - |IN| BAND entries of one target by (exact score
// descending, slot ascending) and set their bits in the LDS bitmap `bm`, then
// compact the bitmap in slot order into the ascending index list (-1 padded).
// Keys: binary64 band scores when `bs` is given, else the fp32 scores.  The
// output is staged in LDS (out_cap ints) when it fits, for coalesced writes.
template <int NT>
__device__ void finish_target(uint32_t *bm, int64_t nwords, int64_t n, int32_t K, int32_t in_cnt, int32_t nb,
                              const int32_t *list, const double *bs, const float *scores_q,
                              const int32_t *cand_q, int32_t *dst, int32_t *count_dst, uint64_t *key_lds,
                              int32_t *slot_lds, int32_t *out_lds, int out_cap, uint32_t *red) {
    const int32_t r = K - in_cnt;
    auto exact_key = [&](int32_t i) -> uint64_t { return dkey(bs ? bs[i] : (double)scores_q[list[i]]); };
    if (r > 0 && nb > 0) {
        if (nb <= BANDFAST) {
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
                    for (int u = 0; u < 16; u++) rank += (kk[u] > ki) || (kk[u] == ki && ss[u] < si);
                }
                for (; j0 < nb; j0++) {
                    const uint64_t kj = key_lds[j0];
                    rank += (kj > ki) || (kj == ki && slot_lds[j0] < si);
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
    __syncthreads();
    const int64_t per = (nwords + NT - 1) / NT;
    const int64_t w0 = (int64_t)threadIdx.x * per;
    uint32_t mine = 0;
    for (int64_t w = w0; w < w0 + per && w < nwords; w++) mine += __builtin_popcount(bm[w]);
    uint32_t tot;
    uint32_t pos = block_excl_scan<NT>(mine, red, tot);
    const bool staged = K <= out_cap;
    for (int64_t w = w0; w < w0 + per && w < nwords; w++) {
        uint32_t bits = bm[w];
        while (bits) {
            const int i = __builtin_ctz(bits);
            bits &= bits - 1;
            const int64_t slot = w * 32 + i;
            if (pos < (uint32_t)K) {
                const int32_t v = cand_q ? cand_q[slot] : (int32_t)slot;
                if (staged) out_lds[pos] = v;
                else dst[pos] = v;
            }
            pos++;
        }
    }
    const uint32_t kept = tot < (uint32_t)K ? tot : (uint32_t)K;
    if (staged) {
        __syncthreads();
        for (int32_t i = threadIdx.x; i < K; i += NT) dst[i] = i < (int32_t)kept ? out_lds[i] : -1;
    } else {
        for (int32_t i = kept + threadIdx.x; i < K; i += NT) dst[i] = -1;
    }
    if (count_dst && threadIdx.x == 0) *count_dst = (int32_t)kept;
    __syncthreads();
}

// ------------------------------------------------------ fused small path
// One 512-thread block per query keeps its n <= 32768 scores in LDS.  With
// the score range known from the indexer's tile statistics, the histogram is
// built while loading; the bin edges of the K-th largest come from a 64-way
// search on the float key space; classification compares in fp32 against
// thresholds rounded outward.  Exact mode also picks the band and compacts
// (one launch); certified mode hands the bitmap and band list on.  Slot s is
// read by thread s % 512, so a wave's 64 consecutive slots give two bitmap
// words straight from one ballot.
constexpr int SMALL_NT = 512;
constexpr int64_t SMALL_N = 32768;
constexpr int SPT = (int)(SMALL_N / SMALL_NT);

struct SmallArgs {
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
};

template <bool CERT>
__global__ __launch_bounds__(SMALL_NT) void k_sel_small(SmallArgs a) {
    __shared__ __attribute__((aligned(16))) float sc[SMALL_N];  // reused by exact mode's finishing step
    __shared__ uint32_t hist[NB];
    __shared__ uint32_t cum[NB + 1];
    __shared__ uint32_t bm[SMALL_N / 32];
    __shared__ uint32_t red[SMALL_NT / 64];
    __shared__ float fred[3][SMALL_NT / 64];
    __shared__ uint32_t grp_sum[SMALL_NT];
    __shared__ int bstar_sh;
    __shared__ uint32_t edge_sh[2];
    __shared__ int32_t band_cnt_sh;
    const int bq = blockIdx.x;
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int n = (int)a.n;
    const int64_t base = (int64_t)bq * a.n;

    for (int i = tid; i < NB; i += SMALL_NT) hist[i] = 0;
    // range (and key norm) from the tile statistics, when given
    float lo = POS_INF, hi = NEG_INF, km = 0.f;
    uint32_t nvalid = 0;
    if (a.stats) {
        uint32_t c = 0;
        for (int t = tid; t < a.ntiles; t += SMALL_NT) {
            const TileStat st = a.stats[(size_t)bq * a.ntiles + t];
            lo = fminf(lo, st.smin);
            hi = fmaxf(hi, st.smax);
            km = fmaxf(km, st.kmax2);
            c += st.nvalid;
        }
        lo = wave_min(lo);
        hi = wave_max(hi);
        km = wave_max(km);
        if (lane == 0) {
            fred[0][wave] = lo;
            fred[1][wave] = hi;
            fred[2][wave] = km;
        }
        nvalid = block_sum_u32<SMALL_NT>(c, red);  // barriers inside
        for (int i = 0; i < SMALL_NT / 64; i++) {
            lo = fminf(lo, fred[0][i]);
            hi = fmaxf(hi, fred[1][i]);
            km = fmaxf(km, fred[2][i]);
        }
    }
    const bool have_range = a.stats != nullptr;
    float inv = (have_range && nvalid > 0 && hi - lo > 0.f) ? (float)NB / (hi - lo) : 0.f;

    // load (8 x 16-byte vectors per thread, all in flight), histogram if the range is known
    {
        constexpr int VPT = SPT / 4;
        f32x4 xv[VPT];
        const f32x4 ninf = {NEG_INF, NEG_INF, NEG_INF, NEG_INF};
        const bool vec_ok = (a.n % 4 == 0) && ((reinterpret_cast<uintptr_t>(a.scores) & 15) == 0);
#pragma unroll
        for (int i = 0; i < VPT; i++) {
            const int s0 = 4 * (tid + SMALL_NT * i);
            if (vec_ok && s0 < n) {
                xv[i] = *reinterpret_cast<const f32x4 *>(a.scores + base + s0);
            } else {
                xv[i] = ninf;
                for (int j = 0; j < 4; j++)
                    if (s0 + j < n) xv[i][j] = a.scores[base + s0 + j];
            }
        }
        if (a.cand) {
            const int32_t *cp = a.cand + base;
#pragma unroll
            for (int i = 0; i < VPT; i++) {
                const int s0 = 4 * (tid + SMALL_NT * i);
                for (int j = 0; j < 4; j++)
                    if (s0 + j < n && cp[s0 + j] < 0) xv[i][j] = NEG_INF;
            }
        }
        float mn = POS_INF, mx = NEG_INF;
        uint32_t cnt = 0;
#pragma unroll
        for (int i = 0; i < VPT; i++) {
            const int s0 = 4 * (tid + SMALL_NT * i);
            *reinterpret_cast<f32x4 *>(sc + s0) = xv[i];
#pragma unroll
            for (int j = 0; j < 4; j++) {
                const float x = xv[i][j];
                if (x != NEG_INF) {
                    if (have_range) {
                        atomicAdd(&hist[sel_bin(x, lo, inv)], 1u);
                    } else {
                        mn = fminf(mn, x);
                        mx = fmaxf(mx, x);
                        cnt++;
                    }
                }
            }
        }
        if (!have_range) {
            mn = wave_min(mn);
            mx = wave_max(mx);
            if (lane == 0) {
                fred[0][wave] = mn;
                fred[1][wave] = mx;
            }
            nvalid = block_sum_u32<SMALL_NT>(cnt, red);
            for (int i = 0; i < SMALL_NT / 64; i++) {
                lo = fminf(lo, fred[0][i]);
                hi = fmaxf(hi, fred[1][i]);
            }
            inv = (nvalid > 0 && hi - lo > 0.f) ? (float)NB / (hi - lo) : 0.f;
#pragma unroll 8
            for (int i = 0; i < SPT; i++) {
                const float x = sc[tid + SMALL_NT * i];
                if (x != NEG_INF) atomicAdd(&hist[sel_bin(x, lo, inv)], 1u);
            }
        }
    }
    __syncthreads();
    // suffix counts: cum[b] = number of scores in bins >= b
    {
        constexpr int BPT = NB / SMALL_NT;
        uint32_t hb[BPT], local = 0;
#pragma unroll
        for (int j = 0; j < BPT; j++) {
            hb[j] = hist[BPT * tid + j];
            local += hb[j];
        }
        grp_sum[SMALL_NT - 1 - tid] = local;
        __syncthreads();
        uint32_t tot;
        const uint32_t ex = block_excl_scan<SMALL_NT>(grp_sum[tid], red, tot);
        __syncthreads();
        grp_sum[tid] = ex;
        __syncthreads();
        uint32_t run = grp_sum[SMALL_NT - 1 - tid];
#pragma unroll
        for (int j = BPT - 1; j >= 0; j--) {
            run += hb[j];
            cum[BPT * tid + j] = run;
        }
        if (tid == 0) cum[NB] = 0;
    }
    // error bound of the fp32 scores (certified mode)
    double E = 0.0;
    if constexpr (CERT)
        E = score_bound(sqrt((double)km * (1.0 + ldexp(1.0, -10))), a.sumwq[bq] * (1.0 + ldexp(1.0, -30)), a.HI,
                        a.dI);
    __syncthreads();

    const int64_t nwords = (a.n + 31) / 32;
    for (int tg = 0; tg < a.ntgt; tg++) {
        const int K = a.K[tg];
        if (tid == 0) {
            bstar_sh = -1;
            band_cnt_sh = 0;
        }
        __syncthreads();
        if (nvalid > (uint32_t)K)
            for (int b2 = (NB / SMALL_NT) * tid; b2 < (NB / SMALL_NT) * (tid + 1); b2++)
                if (cum[b2] >= (uint32_t)K && cum[b2 + 1] < (uint32_t)K) bstar_sh = b2;
        __syncthreads();
        const int bstar = bstar_sh;
        double tlo = -__builtin_inf(), thi = -__builtin_inf();
        if (bstar >= 0) {
            // [a, z] = float values >= lo whose bin is b* (bin() is monotone)
            if (wave == 0) {
                const uint32_t lk = fkey(lo), hk = 0xff7fffffu;
                const uint32_t ka = wave_search_bin(lk, hk, bstar, lo, inv);
                const uint32_t kz = bstar + 1 < NB ? wave_search_bin(lk, hk, bstar + 1, lo, inv) - 1 : hk;
                if (lane == 0) {
                    edge_sh[0] = ka;
                    edge_sh[1] = kz;
                }
            }
            __syncthreads();
            tlo = thr_lo(fkey_inv(edge_sh[0]), E);
            thi = thr_hi(fkey_inv(edge_sh[1]), E);
        }
        // IN: x > thi  <=>  x > f_hi;  BAND: x >= tlo  <=>  x >= f_lo  (x is a float)
        const float f_hi = f32_down(thi), f_lo = f32_up(tlo);
        uint32_t nin = 0;
        int32_t *band = a.band + ((size_t)tg * gridDim.x + bq) * a.band_cap;
#pragma unroll 4
        for (int i = 0; i < SPT; i++) {
            const float x = sc[tid + SMALL_NT * i];
            const bool valid = x != NEG_INF;
            const bool in = valid && x > f_hi;
            const bool bnd = valid && !in && x >= f_lo;
            const uint64_t bal = __ballot(in);
            const uint64_t bb = __ballot(bnd);
            const int word0 = (wave * 64 + SMALL_NT * i) >> 5;
            if (lane == 0) {
                bm[word0] = (uint32_t)bal;
                bm[word0 + 1] = (uint32_t)(bal >> 32);
                nin += (uint32_t)__builtin_popcountll(bal);
            }
            if (bb) {
                int32_t basepos = 0;
                if (lane == 0) basepos = atomicAdd(&band_cnt_sh, (int32_t)__builtin_popcountll(bb));
                basepos = __shfl(basepos, 0);
                if (bnd) {
                    const uint32_t below = __builtin_amdgcn_mbcnt_hi((uint32_t)(bb >> 32),
                                                                     __builtin_amdgcn_mbcnt_lo((uint32_t)bb, 0u));
                    band[basepos + (int32_t)below] = tid + SMALL_NT * i;
                }
            }
        }
        const int32_t in_cnt = (int32_t)block_sum_u32<SMALL_NT>(nin, red);  // barriers inside
        const int32_t nb = band_cnt_sh;
        if constexpr (CERT) {
            uint32_t *gbm = a.bitmap + ((size_t)tg * gridDim.x + bq) * a.nwords;
            for (int64_t wd = tid; wd < nwords; wd += SMALL_NT) gbm[wd] = bm[wd];
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
        } else {
            __threadfence_block();
            __syncthreads();
            uint64_t *key_lds = reinterpret_cast<uint64_t *>(sc);
            int32_t *slot_lds = reinterpret_cast<int32_t *>(key_lds + BANDFAST);
            int32_t *out_lds = slot_lds + BANDFAST;
            const int32_t *list = band;
            int32_t *dst = (tg == 0 ? a.out0 : a.out1) + (size_t)bq * K;
            finish_target<SMALL_NT>(bm, nwords, a.n, K, in_cnt, nb, list, nullptr, a.scores + base,
                                    a.cand ? a.cand + base : nullptr, dst, tg == 0 && a.count0 ? a.count0 + bq : nullptr,
                                    key_lds, slot_lds, out_lds, (int)(SMALL_N - 3 * BANDFAST), red);
        }
        __syncthreads();
    }
}

// ----------------------------------------------------------------- rescore
// One wave per BAND entry (both targets' lists back to back).  The block
// stages its query's indexer heads in LDS as fp32 rows; lane h computes head
// h's dot product with the staged key row in the definition's order d = 0, 1,
// ... (products of bf16/fp32 inputs are exact in binary64, so fma = rounded
// product + add); t_h = w_h * ReLU(d_h) is rounded on its own and the head
// sum runs h = 0, 1, ... from +0.0 through lane broadcasts.  Idle blocks exit
// at once.
constexpr int RS_NT = 256;
constexpr int RS_DMAX = 1024;  // longest key row

struct RescoreKArgs {
    const void *qI;
    int dt;
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
};

__device__ __forceinline__ double readlane_f64(double x, int l) {
    const uint64_t u = __double_as_longlong(x);
    const uint32_t lo = __builtin_amdgcn_readlane((uint32_t)u, l);
    const uint32_t hi = __builtin_amdgcn_readlane((uint32_t)(u >> 32), l);
    return __longlong_as_double(((uint64_t)hi << 32) | lo);
}

__device__ __forceinline__ float ld_elem(const void *p, int dt, size_t i) {
    return dt == CSA2_F32 ? static_cast<const float *>(p)[i] : bf16_to_f32(static_cast<const uint16_t *>(p)[i]);
}

// rows x cols elements (fp32 or bf16, from element `off`) -> fp32 LDS rows of
// `stride` floats; 16-byte loads, four in flight per thread.
template <int NT>
__device__ void stage_rows(float *dst, int stride, const void *src, int dt, size_t off, int rows, int cols) {
    const int total = rows * cols;
    const int esz = dt == CSA2_F32 ? 4 : 2;
    const int per = 16 / esz;  // elements per 16-byte vector
    const char *p = static_cast<const char *>(src) + off * esz;
    const bool vec = ((reinterpret_cast<uintptr_t>(p) & 15) == 0) && (cols % per == 0);
    if (!vec) {
        for (int i = threadIdx.x; i < total; i += NT) {
            const int r = i / cols;
            dst[r * stride + (i - r * cols)] = dt == CSA2_F32 ? reinterpret_cast<const float *>(p)[i]
                                                              : bf16_to_f32(reinterpret_cast<const uint16_t *>(p)[i]);
        }
        return;
    }
    const int nvec = total / per, vpr = cols / per;  // vectors per row
    for (int v0 = threadIdx.x; v0 < nvec; v0 += 4 * NT) {
        u32x4 buf[4];
#pragma unroll
        for (int u = 0; u < 4; u++)
            if (v0 + u * NT < nvec) buf[u] = reinterpret_cast<const u32x4 *>(p)[v0 + u * NT];
#pragma unroll
        for (int u = 0; u < 4; u++) {
            const int vi = v0 + u * NT;
            if (vi >= nvec) continue;
            const int r = vi / vpr;
            float *d = dst + r * stride + (vi - r * vpr) * per;
            if (dt == CSA2_F32) {
#pragma unroll
                for (int x = 0; x < 4; x++) d[x] = __uint_as_float(buf[u][x]);
            } else {
#pragma unroll
                for (int x = 0; x < 8; x++) d[x] = bf16_to_f32((uint16_t)(buf[u][x >> 1] >> (16 * (x & 1))));
            }
        }
    }
}

__global__ __launch_bounds__(RS_NT) void k_sel_rescore(RescoreKArgs a) {
#pragma clang fp contract(off)
    extern __shared__ __attribute__((aligned(16))) float lds[];
    const int bq = blockIdx.y;
    const int b = bq / a.Q;
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    constexpr int NW = RS_NT / 64;
    const SelQuery sqv = a.sq[bq];
    const int32_t nb0 = sqv.t[0].band_cnt, nb1 = a.ntgt > 1 ? sqv.t[1].band_cnt : 0;
    const int32_t total = nb0 + nb1;
    if ((int32_t)blockIdx.x * NW >= total) return;
    const int qstride = a.dI + 1;  // padded rows: lane h reads bank (h + d) % 64
    float *qs = lds;
    float *ks = lds + ((a.HI * qstride + 3) & ~3) + wave * a.dI;
    stage_rows<RS_NT>(qs, qstride, a.qI, a.dt, (size_t)bq * a.HI * a.dI, a.HI, a.dI);
    __syncthreads();
    for (int32_t e = blockIdx.x * NW + wave; e < total; e += gridDim.x * NW) {
        const int tg = e < nb0 ? 0 : 1;
        const int32_t pos = tg == 0 ? e : e - nb0;
        const int32_t slot = a.band[((size_t)tg * gridDim.y + bq) * a.band_cap + pos];
        const int64_t j = a.cand ? (int64_t)a.cand[(int64_t)bq * a.n + slot] : (int64_t)slot;
        {
            float kv[RS_DMAX / 64];
            const size_t kb = ((size_t)b * a.N + j) * a.dI;
#pragma unroll
            for (int u = 0; u < RS_DMAX / 64; u++)
                if (lane + 64 * u < a.dI) kv[u] = ld_elem(a.kI, a.dt, kb + lane + 64 * u);
#pragma unroll
            for (int u = 0; u < RS_DMAX / 64; u++)
                if (lane + 64 * u < a.dI) ks[lane + 64 * u] = kv[u];
        }
        __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
        __builtin_amdgcn_wave_barrier();
        __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
        double s = 0.0;
        for (int h0 = 0; h0 < a.HI; h0 += 64) {
            const int h = h0 + lane;
            double t = 0.0;
            if (h < a.HI) {
                const float *qh = qs + h * qstride;
                double dot = 0.0;
                int d0 = 0;
                for (; d0 + 8 <= a.dI; d0 += 8) {
                    float qv[8], kk[8];
#pragma unroll
                    for (int u = 0; u < 8; u++) {
                        qv[u] = qh[d0 + u];
                        kk[u] = ks[d0 + u];
                    }
#pragma unroll
                    for (int u = 0; u < 8; u++) dot = __builtin_fma((double)qv[u], (double)kk[u], dot);
                }
                for (; d0 < a.dI; d0++) dot = __builtin_fma((double)qh[d0], (double)ks[d0], dot);
                const double rl = dot > 0.0 ? dot : 0.0;
                t = (double)a.w[(size_t)bq * a.HI + h] * rl;
            }
            const int hn = a.HI - h0 < 64 ? a.HI - h0 : 64;
            for (int i = 0; i < hn; i++) s = s + readlane_f64(t, i);
        }
        if (lane == 0) a.band_score[((size_t)tg * gridDim.y + bq) * a.band_cap + pos] = s;
        __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
        __builtin_amdgcn_wave_barrier();
        __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
    }
}

// ------------------------------------------------------------------ finish
// One block per query: band pick + compaction for each target, the bitmap
// staged in LDS when it fits.
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
};

__global__ __launch_bounds__(FIN_NT) void k_sel_finish(FinishArgs a) {
    __shared__ uint32_t bm_lds[FIN_BM];
    __shared__ uint64_t key_lds[BANDFAST];
    __shared__ int32_t slot_lds[BANDFAST];
    __shared__ int32_t out_lds[FIN_OUT];
    __shared__ uint32_t red[FIN_NT / 64];
    const int bq = blockIdx.x;
    const SelQuery sqv = a.sq[bq];
    for (int tg = 0; tg < a.ntgt; tg++) {
        const SelTarget t = sqv.t[tg];
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
                              key_lds, slot_lds, out_lds, FIN_OUT, red);
    }
}

}  // namespace

// ------------------------------------------------------------------ host

size_t rescore_lds_bytes(int HI, int dI) {
    if (dI > RS_DMAX) return SIZE_MAX;
    return sizeof(float) * ((((size_t)HI * (dI + 1)) + 3) / 4 * 4 + (size_t)(RS_NT / 64) * dI);
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

static bool small_path(const SelPlan &p) { return p.n <= SMALL_N; }

size_t sel_workspace(const SelPlan &p, bool own_stats) {
    Carve c(nullptr, 0);
    if (own_stats && !small_path(p)) c.take<TileStat>((size_t)p.BQ * p.ntiles);
    c.take<uint32_t>((size_t)p.BQ * p.nchunks * NB);
    c.take<SelQuery>((size_t)p.BQ);
    c.take<double>((size_t)p.BQ);  // error bounds
    c.take<uint32_t>((size_t)p.ntgt * p.BQ * p.nwords);
    c.take<int32_t>((size_t)p.ntgt * p.BQ * p.band_cap);
    if (p.certified) c.take<double>((size_t)p.ntgt * p.BQ * p.band_cap);
    return c.used;
}

void sel_run(const SelPlan &p, const float *scores, const int32_t *cand, const TileStat *stats_in,
             const RescoreArgs *rs, int32_t *out0, int32_t *count0, int32_t *out1, void *ws, size_t ws_bytes,
             hipStream_t s) {
    Carve c(ws, ws_bytes);
    TileStat *stats = const_cast<TileStat *>(stats_in);
    if (!stats && !small_path(p)) stats = c.take<TileStat>((size_t)p.BQ * p.ntiles);
    uint32_t *part = c.take<uint32_t>((size_t)p.BQ * p.nchunks * NB);
    SelQuery *sq = c.take<SelQuery>((size_t)p.BQ);
    double *ebuf = c.take<double>((size_t)p.BQ);
    uint32_t *bitmap = c.take<uint32_t>((size_t)p.ntgt * p.BQ * p.nwords);
    int32_t *band = c.take<int32_t>((size_t)p.ntgt * p.BQ * p.band_cap);
    double *band_score = p.certified ? c.take<double>((size_t)p.ntgt * p.BQ * p.band_cap) : nullptr;
    if (c.used > ws_bytes) throw Error(CSA2_EWORKSPACE, "selection workspace too small");
    if (p.certified && (!rs || !rs->sumwq)) throw Error(CSA2_EINTERNAL, "certified selection needs query norms");

    if (small_path(p)) {
        SmallArgs a{};
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
        if (p.certified) hipLaunchKernelGGL(k_sel_small<true>, dim3(p.BQ), dim3(SMALL_NT), 0, s, a);
        else hipLaunchKernelGGL(k_sel_small<false>, dim3(p.BQ), dim3(SMALL_NT), 0, s, a);
        check_launch("selection (fused)");
        if (!p.certified) return;
    } else {
        if (!stats_in) {
            hipLaunchKernelGGL(k_sel_stats, dim3(p.ntiles, p.BQ), dim3(256), 0, s, scores, cand, p.n, p.ntiles,
                               stats);
            check_launch("selection stats");
        }
        if (p.certified)
            launch_err_bound_from_norms(rs->sumwq, p.BQ, rs->HI, rs->dI, stats, p.ntiles, ebuf, s);
        hipLaunchKernelGGL(k_sel_hist, dim3(p.nchunks, p.BQ), dim3(256), 0, s, scores, cand, p.n, stats, p.ntiles,
                           p.nchunks, part, sq);
        check_launch("selection histogram");
        hipLaunchKernelGGL(k_sel_find, dim3(p.BQ), dim3(256), 0, s, part, p.nchunks, p.K0, p.K1,
                           p.certified ? ebuf : nullptr, sq);
        check_launch("selection find");
        const int nblk = (int)((p.nwords + 255) / 256);
        hipLaunchKernelGGL(k_sel_classify, dim3(nblk, p.BQ), dim3(256), 0, s, scores, cand, p.n, p.ntgt, sq, bitmap,
                           p.nwords, band, p.band_cap);
        check_launch("selection classify");
    }
    if (p.certified) {
        RescoreKArgs r{};
        r.qI = rs->qI;
        r.dt = rs->dt;
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
        int nblk = 4096 / p.BQ / (RS_NT / 64);
        nblk = nblk < 2 ? 2 : (nblk > 64 ? 64 : nblk);
        hipLaunchKernelGGL(k_sel_rescore, dim3(nblk, p.BQ), dim3(RS_NT), rescore_lds_bytes(rs->HI, rs->dI), s, r);
        check_launch("selection rescore");
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
    hipLaunchKernelGGL(k_sel_finish, dim3(p.BQ), dim3(FIN_NT), 0, s, f);
    check_launch("selection finish");
}

}  // namespace csa2
