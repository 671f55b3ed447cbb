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
void launch_err_bound(const void *qI, int dt, const float *w, int BQ, int HI, int dI, const TileStat *stats,
                      int ntiles, float *err32, double *err64, hipStream_t s);
void launch_err_bound_from_norms(const double *sumwq, int BQ, int HI, int dI, const TileStat *stats, int ntiles,
                                 double *err64, hipStream_t s);

// -------------------------------------------------------------- selection
struct SelPlan {
    int BQ;
    int64_t n;
    int K0, K1;  // top-k and (0 or) pool size
    int ntgt, ntiles, nchunks;
    int64_t nwords, band_cap;
    bool certified;
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
void sel_run(const SelPlan &p, const float *scores, const int32_t *cand, const TileStat *stats,
             const RescoreArgs *rs, int32_t *out0, int32_t *count0, int32_t *out1, void *ws, size_t ws_bytes,
             hipStream_t s);

// -------------------------------------------------------------- attention
struct AttnPlan {
    int q_dt, kv_dt;
    int B, Q, H, D;
    int64_t N;
    int k;
    bool mfma;
    int nsplit;
};
AttnPlan attn_plan(int q_dt, int kv_dt, int B, int Q, int H, int D, int64_t N, int k);
bool attn_supported(const AttnPlan &p);
size_t attn_workspace(const AttnPlan &p);
void attn_run(const AttnPlan &p, const void *q, const void *kv, const int32_t *idx, float scale, void *out,
              float *lse, void *ws, size_t ws_bytes, hipStream_t s);

// ------------------------------------------------------------ compression
size_t compress_workspace(int dt, int64_t n_out, int D, int m, int halo);
void compress_run(const void *x, int dt, int64_t n_out, int D, int m, int halo, const void *wz, const float *bias,
                  void *out, void *ws, size_t ws_bytes, hipStream_t s);

}  // namespace csa2
