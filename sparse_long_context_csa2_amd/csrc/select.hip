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
                if (E > 0.0) {
                    const double marg = 2.0 * E * (1.0 + ldexp(1.0, -20));
                    t.lo = (double)a - marg - fabs((double)a) * ldexp(1.0, -50);
                    t.hi = (double)z + marg + fabs((double)z) * ldexp(1.0, -50);
                } else {
                    t.lo = (double)a;
                    t.hi = (double)z;
                }
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

// ------------------------------------------------------------- 4: rescore
// One wave per BAND entry; lanes are indexer heads.  Query heads are staged in
// LDS as fp32 (exact for bf16/fp32 inputs); the key row is staged per wave.
__global__ __launch_bounds__(256) void k_sel_rescore(const void *__restrict__ qI, int dt, const float *__restrict__ w,
                                                     const void *__restrict__ kI, int Q, int HI, int dI, int64_t N,
                                                     const int32_t *__restrict__ cand, int64_t n,
                                                     const SelQuery *__restrict__ sq, const int32_t *__restrict__ band,
                                                     int64_t band_cap, double *__restrict__ band_score) {
#pragma clang fp contract(off)
    extern __shared__ float lds[];
    const int bq = blockIdx.y, tgt = blockIdx.z;
    const int b = bq / Q;
    const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
    const int qstride = dI + 1;  // padded row: lane h reads bank (h + d) % 64
    float *qs = lds;
    float *ks = lds + HI * qstride + wave * dI;
    const int toff = (HI * qstride + 4 * dI + 1) & ~1;  // 8-byte aligned start of the per-wave fp64 buffers
    double *ts = reinterpret_cast<double *>(lds + toff) + wave * 64;
    for (int i = threadIdx.x; i < HI * dI; i += 256) {
        int h = i / dI, d = i % dI;
        size_t off = (size_t)bq * HI * dI + i;
        qs[h * qstride + d] = dt == CSA2_F32 ? static_cast<const float *>(qI)[off]
                                             : bf16_to_f32(static_cast<const uint16_t *>(qI)[off]);
    }
    __syncthreads();
    const int32_t cnt = sq[bq].t[tgt].band_cnt;
    const int32_t *list = band + ((size_t)tgt * gridDim.y + bq) * band_cap;
    double *out = band_score + ((size_t)tgt * gridDim.y + bq) * band_cap;
    for (int32_t e = blockIdx.x * 4 + wave; e < cnt; e += gridDim.x * 4) {
        const int32_t slot = list[e];
        const int64_t j = cand ? (int64_t)cand[(int64_t)bq * n + slot] : (int64_t)slot;
        const size_t kbase = ((size_t)b * N + j) * dI;
        for (int d = lane; d < dI; d += 64)
            ks[d] = dt == CSA2_F32 ? static_cast<const float *>(kI)[kbase + d]
                                   : bf16_to_f32(static_cast<const uint16_t *>(kI)[kbase + d]);
        __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
        __builtin_amdgcn_wave_barrier();
        __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
        double s = 0.0;
        for (int h0 = 0; h0 < HI; h0 += 64) {
            const int h = h0 + lane;
            double t = 0.0;
            if (h < HI) {
                double dot = 0.0;
                const float *qh = qs + h * qstride;
                for (int d = 0; d < dI; d++) dot = __builtin_fma((double)qh[d], (double)ks[d], dot);
                const double r = dot > 0.0 ? dot : 0.0;
                t = (double)w[(size_t)bq * HI + h] * r;
            }
            ts[lane] = t;
            __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
            __builtin_amdgcn_wave_barrier();
            __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
            const int hn = HI - h0 < 64 ? HI - h0 : 64;
            for (int i = 0; i < hn; i++) s = s + ts[i];
            __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
            __builtin_amdgcn_wave_barrier();
            __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
        }
        if (lane == 0) out[e] = s;
    }
}

// --------------------------------------------------- 5: band pick + compact
__device__ __forceinline__ uint32_t load_word(const uint32_t *p) {
    return __hip_atomic_load(p, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

__global__ __launch_bounds__(1024) void k_sel_finish(const float *__restrict__ scores,
                                                     const int32_t *__restrict__ cand, int64_t n, int ntgt,
                                                     const SelQuery *__restrict__ sq, uint32_t *__restrict__ bitmap,
                                                     int64_t nwords, const int32_t *__restrict__ band,
                                                     const double *__restrict__ band_score, int64_t band_cap,
                                                     int32_t *__restrict__ out0, int32_t *__restrict__ count0,
                                                     int32_t *__restrict__ out1) {
    __shared__ uint64_t key[BANDFAST];
    __shared__ int32_t bslot[BANDFAST];
    __shared__ uint32_t red[16];
    const int bq = blockIdx.x;
    const int BQ = gridDim.x;
    const int64_t base = (int64_t)bq * n;
    for (int tgt = 0; tgt < ntgt; tgt++) {
        const SelTarget t = sq[bq].t[tgt];
        uint32_t *bm = bitmap + ((size_t)tgt * BQ + bq) * nwords;
        const int32_t *list = band + ((size_t)tgt * BQ + bq) * band_cap;
        const double *bs = band_score ? band_score + ((size_t)tgt * BQ + bq) * band_cap : nullptr;
        const int32_t r = t.K - t.in_cnt;
        const int32_t nb = t.band_cnt;
        auto exact_key = [&](int32_t i) -> uint64_t {
            return dkey(bs ? bs[i] : (double)scores[base + list[i]]);
        };
        if (r > 0 && nb > 0) {
            if (nb <= BANDFAST) {
                for (int32_t i = threadIdx.x; i < nb; i += 1024) {
                    key[i] = exact_key(i);
                    bslot[i] = list[i];
                }
                __syncthreads();
                for (int32_t i = threadIdx.x; i < nb; i += 1024) {
                    const uint64_t ki = key[i];
                    const int32_t si = bslot[i];
                    int32_t rank = 0;
                    for (int32_t j = 0; j < nb; j++) {
                        const uint64_t kj = key[j];
                        rank += (kj > ki) || (kj == ki && bslot[j] < si);
                    }
                    if (rank < r) atomicOr(&bm[si >> 5], 1u << (si & 31));
                }
            } else {
                // bisection on the key for the r-th best, then on the slot among ties
                uint64_t L = 0, R = ~0ull;
                while (L < R) {
                    const uint64_t M = L + (R - L) / 2 + 1;  // count(key >= M) >= r ?
                    uint32_t c = 0;
                    for (int32_t i = threadIdx.x; i < nb; i += 1024) c += exact_key(i) >= M;
                    c = block_sum_u32<1024>(c, red);
                    if (c >= (uint32_t)r) L = M;
                    else R = M - 1;
                }
                const uint64_t tau = L;
                uint32_t gt = 0;
                for (int32_t i = threadIdx.x; i < nb; i += 1024) gt += exact_key(i) > tau;
                gt = block_sum_u32<1024>(gt, red);
                const uint32_t need = (uint32_t)r - gt;
                int64_t SL = 0, SR = n - 1;  // smallest slot bound with count(key==tau, slot<=bound) >= need
                while (SL < SR) {
                    const int64_t M = SL + (SR - SL) / 2;
                    uint32_t c = 0;
                    for (int32_t i = threadIdx.x; i < nb; i += 1024) c += (exact_key(i) == tau) && (list[i] <= M);
                    c = block_sum_u32<1024>(c, red);
                    if (c >= need) SR = M;
                    else SL = M + 1;
                }
                for (int32_t i = threadIdx.x; i < nb; i += 1024) {
                    const uint64_t k = exact_key(i);
                    const int32_t s = list[i];
                    if (k > tau || (k == tau && s <= SL)) atomicOr(&bm[s >> 5], 1u << (s & 31));
                }
            }
        }
        __threadfence();
        __syncthreads();
        // compaction in slot order
        const int64_t per = (nwords + 1023) / 1024;
        const int64_t w0 = (int64_t)threadIdx.x * per;
        uint32_t mine = 0;
        for (int64_t w = w0; w < w0 + per && w < nwords; w++) mine += __builtin_popcount(load_word(bm + w));
        uint32_t tot;
        uint32_t pos = block_excl_scan<1024>(mine, red, tot);
        const int32_t K = t.K;
        int32_t *dst = (tgt == 0 ? out0 : out1) + (size_t)bq * K;
        for (int64_t w = w0; w < w0 + per && w < nwords; w++) {
            uint32_t bits = load_word(bm + w);
            while (bits) {
                const int i = __builtin_ctz(bits);
                bits &= bits - 1;
                const int64_t slot = w * 32 + i;
                if (pos < (uint32_t)K) dst[pos] = cand ? cand[base + slot] : (int32_t)slot;
                pos++;
            }
        }
        const uint32_t kept = tot < (uint32_t)K ? tot : (uint32_t)K;
        for (int32_t i = kept + threadIdx.x; i < K; i += 1024) dst[i] = -1;
        if (tgt == 0 && count0 && threadIdx.x == 0) count0[bq] = (int32_t)kept;
        __syncthreads();
    }
}

}  // namespace

// ------------------------------------------------------------------ host

size_t rescore_lds_bytes(int HI, int dI) {
    const size_t floats = ((size_t)HI * (dI + 1) + 4 * (size_t)dI + 1) & ~size_t(1);
    return sizeof(float) * floats + sizeof(double) * 4 * 64;
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

size_t sel_workspace(const SelPlan &p, bool own_stats) {
    Carve c(nullptr, 0);
    if (own_stats) c.take<TileStat>((size_t)p.BQ * p.ntiles);
    c.take<uint32_t>((size_t)p.BQ * p.nchunks * NB);
    c.take<SelQuery>((size_t)p.BQ);
    c.take<uint32_t>((size_t)p.ntgt * p.BQ * p.nwords);
    c.take<int32_t>((size_t)p.ntgt * p.BQ * p.band_cap);
    if (p.certified) c.take<double>((size_t)p.ntgt * p.BQ * p.band_cap);
    return c.used;
}

void sel_run(const SelPlan &p, const float *scores, const int32_t *cand, const TileStat *stats_in,
             const double *ebound, const RescoreArgs *rs, int32_t *out0, int32_t *count0, int32_t *out1, void *ws,
             size_t ws_bytes, hipStream_t s) {
    Carve c(ws, ws_bytes);
    TileStat *stats = const_cast<TileStat *>(stats_in);
    if (!stats) stats = c.take<TileStat>((size_t)p.BQ * p.ntiles);
    uint32_t *part = c.take<uint32_t>((size_t)p.BQ * p.nchunks * NB);
    SelQuery *sq = c.take<SelQuery>((size_t)p.BQ);
    uint32_t *bitmap = c.take<uint32_t>((size_t)p.ntgt * p.BQ * p.nwords);
    int32_t *band = c.take<int32_t>((size_t)p.ntgt * p.BQ * p.band_cap);
    double *band_score = p.certified ? c.take<double>((size_t)p.ntgt * p.BQ * p.band_cap) : nullptr;
    if (c.used > ws_bytes) throw Error(CSA2_EWORKSPACE, "selection workspace too small");

    if (!stats_in) {
        hipLaunchKernelGGL(k_sel_stats, dim3(p.ntiles, p.BQ), dim3(256), 0, s, scores, cand, p.n, p.ntiles, stats);
        check_launch("selection stats");
    }
    hipLaunchKernelGGL(k_sel_hist, dim3(p.nchunks, p.BQ), dim3(256), 0, s, scores, cand, p.n, stats, p.ntiles,
                       p.nchunks, part, sq);
    check_launch("selection histogram");
    hipLaunchKernelGGL(k_sel_find, dim3(p.BQ), dim3(256), 0, s, part, p.nchunks, p.K0, p.K1,
                       p.certified ? ebound : nullptr, sq);
    check_launch("selection find");
    const int nblk = (int)((p.nwords + 255) / 256);
    hipLaunchKernelGGL(k_sel_classify, dim3(nblk, p.BQ), dim3(256), 0, s, scores, cand, p.n, p.ntgt, sq, bitmap,
                       p.nwords, band, p.band_cap);
    check_launch("selection classify");
    if (p.certified) {
        int per_q = 4096 / p.BQ;
        per_q = per_q < 1 ? 1 : (per_q > 64 ? 64 : per_q);
        const size_t lds = rescore_lds_bytes(rs->HI, rs->dI);
        hipLaunchKernelGGL(k_sel_rescore, dim3(per_q, p.BQ, p.ntgt), dim3(256), lds, s, rs->qI, rs->dt, rs->w, rs->kI,
                           rs->Q, rs->HI, rs->dI, rs->N, cand, p.n, sq, band, p.band_cap, band_score);
        check_launch("selection rescore");
    }
    hipLaunchKernelGGL(k_sel_finish, dim3(p.BQ), dim3(1024), 0, s, scores, cand, p.n, p.ntgt, sq, bitmap, p.nwords,
                       band, band_score, p.band_cap, out0, count0, out1);
    check_launch("selection finish");
}

}  // namespace csa2
