// Internal launch interfaces between the C-ABI host code and the kernels.
#pragma once

#include "common.h"

namespace csa2 {

// ---------------------------------------------------------------- indexer
bool index_mfma_supported(int dt, int HI, int dI);
bool index_valu_supported(int HI, int dI);
void launch_index_score(const void *qI, int dt, const float *w, const void *kI, int B, int Q, int HI, int dI,
                        int64_t N, const int64_t *q_pos, int m, const int32_t *cand, int P, float *scores,
                        TileStat *stats, double *sumwq, hipStream_t s);
// FP4 rows (D channels, D % 64 == 0, 4-byte aligned) decoded exactly to bf16 [nrows][D].
void launch_fp4_rows_to_bf16(const void *rows, int64_t nrows, int D, uint16_t *out, hipStream_t s);
void launch_err_bound(const void *qI, int dt, const float *w, int BQ, int HI, int dI, const TileStat *stats,
                      int ntiles, float *err32, double *err64, hipStream_t s);

// -------------------------------------------------------------- selection
// Per-query selection records (certified mode): for each target, the value
// interval of the band, K, |IN| and |BAND|.
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
// What a certified selection leaves for its top-k target when the final pick
// and compaction are left to the consumer (the attention kernel): the IN
// entries in ascending order, the IN bitmap, the band list with its binary64
// scores, and where the ascending index list and its count go.
struct SelHandoff {
    const SelQuery *sq;
    const int32_t *in_list;  // [BQ][in_cap] IN entries of target 0, ascending
    int64_t in_cap;
    const uint32_t *bitmap;  // [BQ][nwords] IN bits of target 0
    int64_t nwords;
    const int32_t *band;     // [BQ][band_cap] band slots of target 0
    const double *band_score;
    int64_t band_cap;
    const int32_t *cand;     // slot -> entry (nullable)
    int64_t n;               // slots per query
    int32_t *idx;            // [BQ][K] out
    int32_t *count;          // [BQ] out, nullable
};
struct SelPlan {
    int BQ;
    int64_t n;
    int K0, K1;  // top-k and (0 or) pool size
    int ntgt, ntiles, nchunks;
    int64_t nwords, band_cap;
    bool certified;
    bool bf16key = false;  // certified: rank the binary64 scores rounded to bfloat16
};
struct RescoreArgs {
    const void *qI;
    int dt;
    const float *w;
    const void *kI;
    int Q, HI, dI;
    int64_t N;
    const double *sumwq;  // [BQ] sum_h |w_h| ||q_h|| written by the indexer
};
bool rescore_supported(int dt, int dI);  // rows of whole 16-byte vectors
SelPlan sel_plan(int BQ, int64_t n, int K0, int K1, bool certified);
size_t sel_workspace(const SelPlan &p, bool own_stats);
// With `handoff` (certified mode only) the top-k target is not finished here:
// the records it needs are described in *handoff (out0/count0 are stored
// there as the destinations) and the pool target, if any, is finished.
void sel_run(const SelPlan &p, const float *scores, const int32_t *cand, const TileStat *stats,
             const RescoreArgs *rs, int32_t *out0, int32_t *count0, int32_t *out1, void *ws, size_t ws_bytes,
             hipStream_t s, SelHandoff *handoff = nullptr);
bool sel_handoff_supported(const SelPlan &p);

// -------------------------------------------------------------- attention
struct AttnPlan {
    int q_dt, kv_dt;
    int B, Q, H, D;
    int64_t N;
    int k;
    bool mfma;
    int nsplit;
    bool tiles;  // prefill chunk: whole queries per block over 64-row tiles
};
AttnPlan attn_plan(int q_dt, int kv_dt, int B, int Q, int H, int D, int64_t N, int k);
bool attn_supported(const AttnPlan &p);
size_t attn_workspace(const AttnPlan &p);
// With `sel`, the selected entries come from a certified selection's records
// (the top-k target finished in the kernel: each block derives its own split,
// and one block per query writes sel->idx / sel->count) instead of from idx.
void attn_run(const AttnPlan &p, const void *q, const void *kv, const int32_t *idx, float scale, void *out,
              float *lse, void *ws, size_t ws_bytes, hipStream_t s, const SelHandoff *sel = nullptr);
bool attn_handoff_supported(const AttnPlan &p, const SelPlan &sp);

// ------------------------------------------------------------ compression
size_t compress_workspace(int dt, int64_t n_out, int D, int m, int halo);
void compress_run(const void *x, int dt, int64_t n_out, int D, int m, int halo, const void *wz, const float *bias,
                  void *out, void *ws, size_t ws_bytes, hipStream_t s);

// ------------------------------------------------------------- SWA branch
void launch_window_idx(const int64_t *q_pos, int64_t BQ, int W, int64_t T, int32_t *idx, hipStream_t s);
void launch_merge_attn(int dt, const void *oa, const float *la, const void *ob, const float *lb, int64_t R, int D,
                       void *out, float *lse, hipStream_t s);

// ------------------------------------------------------- FP4 cache writes
void launch_quantize_fp4(const void *x, int dt, int64_t n, int D, uint8_t *cache, const int64_t *dst_row,
                         hipStream_t s);

}  // namespace csa2
