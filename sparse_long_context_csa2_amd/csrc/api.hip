// C ABI of the CSA2 hot path (include/csa2.h): argument validation before any
// launch, workspace carving and the Full / Reindex / Reuse mode sequencing.
#include <cstring>
#include <mutex>
#include <string>

#include "internal.h"

namespace {

thread_local std::string g_last_error;

using csa2::Error;

bool aligned16(const void *p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

void need_ptr(const void *p, const char *name) {
    if (!p) throw Error(CSA2_EINVAL, std::string(name) + " is NULL");
    if (!aligned16(p)) throw Error(CSA2_EINVAL, std::string(name) + " is not 16-byte aligned");
}
void opt_ptr(const void *p, const char *name) {
    if (p && !aligned16(p)) throw Error(CSA2_EINVAL, std::string(name) + " is not 16-byte aligned");
}
void need_ws(void *ws, size_t ws_bytes, size_t need) {
    if (ws_bytes < need) throw Error(CSA2_EWORKSPACE, "workspace has " + std::to_string(ws_bytes) + " bytes, needs " +
                                                          std::to_string(need));
    if (need && !ws) throw Error(CSA2_EINVAL, "workspace is NULL");
    if (ws && (reinterpret_cast<uintptr_t>(ws) & 255u)) throw Error(CSA2_EINVAL, "workspace is not 256-byte aligned");
}
void need_plain_dt(int dt, const char *name) {
    if (dt != CSA2_F32 && dt != CSA2_BF16) throw Error(CSA2_EINVAL, std::string(name) + " must be CSA2_F32 or CSA2_BF16");
}

template <class F>
int guarded(F &&f) {
    try {
        f();
        return CSA2_OK;
    } catch (const Error &e) {
        g_last_error = e.what();
        return e.code;
    } catch (const std::exception &e) {
        g_last_error = e.what();
        return CSA2_EINTERNAL;
    } catch (...) {
        g_last_error = "unknown failure";
        return CSA2_EINTERNAL;
    }
}

// Queries (B * Q) index the second grid dimension of the indexer, selection
// and vector-attention launches: checked here, before anything is enqueued.
constexpr int64_t MAX_QUERIES = 65535;
void check_queries(int32_t B, int32_t Q) {
    if ((int64_t)B * Q > MAX_QUERIES)
        throw Error(CSA2_EUNSUPPORTED, "B * Q = " + std::to_string((int64_t)B * Q) + " query rows; at most " +
                                           std::to_string(MAX_QUERIES) + " per call");
}

// ------------------------------------------------------------- indexer
// FP4 queries are decoded into bf16 in the workspace first; the kernels then
// see FP4 keys with bf16 queries.
int kernel_idx_dt(int dt) { return dt == CSA2_FP4QK ? CSA2_FP4 : dt; }
size_t qdec_bytes(int dt, int32_t B, int32_t Q, int32_t HI, int32_t dI) {
    return dt == CSA2_FP4QK ? (size_t)B * Q * HI * dI * 2 : 0;
}
const void *decode_queries(const void *qI, int dt, int32_t B, int32_t Q, int32_t HI, int32_t dI, csa2::Carve &c,
                           hipStream_t s) {
    if (dt != CSA2_FP4QK) return qI;
    uint16_t *qd = c.take<uint16_t>((size_t)B * Q * HI * dI);
    csa2::launch_fp4_rows_to_bf16(qI, (int64_t)B * Q * HI, dI, qd, s);
    return qd;
}

void check_index_args(int dt0, int32_t B, int32_t Q, int32_t HI, int32_t dI, int64_t N, int32_t P) {
    const int dt = kernel_idx_dt(dt0);
    if (dt != CSA2_FP4) need_plain_dt(dt, "indexer dtype");
    if (dt == CSA2_FP4 && !csa2::index_mfma_supported(dt, HI, dI))
        throw Error(CSA2_EUNSUPPORTED, "FP4 indexer keys need a matrix-core shape with dI % 64 == 0");
    if (B < 1 || Q < 1 || HI < 1 || dI < 1 || N < 1) throw Error(CSA2_EINVAL, "B, Q, HI, dI and N must be >= 1");
    if (N > INT32_MAX || P < 0) throw Error(CSA2_EINVAL, "N must fit int32 and P must be >= 0");
    check_queries(B, Q);
    if (!csa2::index_mfma_supported(dt, HI, dI) && !csa2::index_valu_supported(HI, dI))
        throw Error(CSA2_EUNSUPPORTED, "no indexer kernel for HI*dI > 16384 with this shape");
    if (dt == CSA2_BF16 && dI % 8) throw Error(CSA2_EINVAL, "bf16 indexer rows need dI % 8 == 0");
}

size_t index_ws(int dt, int32_t B, int32_t Q, int32_t HI, int32_t dI, int64_t n) {
    csa2::Carve c(nullptr, 0);
    c.take<csa2::TileStat>((size_t)B * Q * ((n + csa2::TILE - 1) / csa2::TILE));
    if (dt == CSA2_FP4QK) c.take<uint16_t>(qdec_bytes(dt, B, Q, HI, dI) / 2);
    return c.used;
}

// --------------------------------------------------------------- layer
struct LayerSizes {
    int64_t n;  // scored slots per query
    csa2::SelPlan sel;
    csa2::AttnPlan att;
    size_t scores, stats, selws, attws, total;
};

LayerSizes layer_sizes(const csa2_layer_args *a) {
    LayerSizes z{};
    const int BQ = a->B * a->Q;
    z.att = csa2::attn_plan(a->q_dt, a->kv_dt, a->B, a->Q, a->H, a->D, a->N, a->k);
    z.attws = csa2::attn_workspace(z.att);
    if (a->mode == CSA2_REUSE) {
        z.total = z.attws;
        return z;
    }
    z.n = a->mode == CSA2_FULL ? a->N : a->P;
    z.sel = csa2::sel_plan(BQ, z.n, a->k, a->mode == CSA2_FULL ? a->P : 0, true);
    z.sel.bf16key = a->score_fmt == CSA2_SCORE_BF16;
    csa2::Carve c(nullptr, 0);
    z.scores = a->scores ? 0 : (c.take<float>((size_t)BQ * z.n), (size_t)BQ * z.n * 4);
    size_t before = c.used;
    c.take<csa2::TileStat>((size_t)BQ * z.sel.ntiles);
    c.take<double>((size_t)BQ);  // sum_h |w_h| ||q_h||
    if (a->idx_dt == CSA2_FP4QK) c.take<uint16_t>(qdec_bytes(a->idx_dt, a->B, a->Q, a->HI, a->dI) / 2);
    z.stats = c.used - before;
    z.selws = csa2::sel_workspace(z.sel, false);
    z.total = c.used + z.selws + z.attws;
    return z;
}

void check_layer(const csa2_layer_args *a) {
    if (!a) throw Error(CSA2_EINVAL, "args is NULL");
    if (a->mode != CSA2_FULL && a->mode != CSA2_REINDEX && a->mode != CSA2_REUSE)
        throw Error(CSA2_EINVAL, "unknown mode");
    if (a->B < 1 || a->Q < 1 || a->N < 1 || a->k < 1 || a->H < 1 || a->D < 1)
        throw Error(CSA2_EINVAL, "B, Q, N, k, H and D must be >= 1");
    check_queries(a->B, a->Q);
    need_ptr(a->q, "q");
    need_ptr(a->kv, "kv");
    need_ptr(a->out, "out");
    opt_ptr(a->lse, "lse");
    opt_ptr(a->count, "count");
    need_ptr(a->idx, "idx");
    need_plain_dt(a->q_dt, "q dtype");
    if (a->kv_dt != CSA2_F32 && a->kv_dt != CSA2_BF16 && a->kv_dt != CSA2_FP4)
        throw Error(CSA2_EINVAL, "unknown kv format");
    if (a->kv_dt == CSA2_FP4 && (a->D % 16 || a->q_dt != CSA2_BF16))
        throw Error(CSA2_EINVAL, "FP4 kv needs D % 16 == 0 and bf16 queries");
    if (a->kv_dt == CSA2_BF16 && a->D % 8) throw Error(CSA2_EINVAL, "bf16 kv rows need D % 8 == 0");
    if (!csa2::attn_supported(csa2::attn_plan(a->q_dt, a->kv_dt, a->B, a->Q, a->H, a->D, a->N, a->k)))
        throw Error(CSA2_EUNSUPPORTED, "no attention kernel for this shape (vector path needs D + k <= 16384)");
    if (a->mode == CSA2_REUSE) return;
    if (a->score_fmt != CSA2_SCORE_F64 && a->score_fmt != CSA2_SCORE_BF16) throw Error(CSA2_EINVAL, "unknown score_fmt");
    need_ptr(a->qI, "qI");
    if (a->idx_dt == CSA2_FP4QK && (reinterpret_cast<uintptr_t>(a->qI) & 3))
        throw Error(CSA2_EINVAL, "FP4 query rows must be 4-byte aligned");
    need_ptr(a->w, "w");
    need_ptr(a->kI, "kI");
    opt_ptr(a->scores, "scores");
    opt_ptr(a->q_pos, "q_pos");
    if (a->q_pos && a->m < 1) throw Error(CSA2_EINVAL, "m must be >= 1 with q_pos");
    if (!csa2::rescore_supported(kernel_idx_dt(a->idx_dt), a->dI))
        throw Error(CSA2_EUNSUPPORTED, "certified selection needs indexer rows of whole 16-byte vectors "
                                       "(dI % 4 == 0 for fp32, dI % 8 == 0 for bf16, dI % 64 == 0 and "
                                       "dI <= 256 for FP4 keys)");
    if (a->mode == CSA2_FULL) {
        if (a->P < 0) throw Error(CSA2_EINVAL, "P must be >= 0");
        if (a->P > 0) need_ptr(a->pool, "pool");
        check_index_args(a->idx_dt, a->B, a->Q, a->HI, a->dI, a->N, a->P);
    } else {
        if (a->P < 1) throw Error(CSA2_EINVAL, "REINDEX needs P >= 1 pool slots");
        need_ptr(a->pool, "pool");
        check_index_args(a->idx_dt, a->B, a->Q, a->HI, a->dI, a->N, a->P);
    }
}

// The layer's launches, with scratch carved from ws (at least z.total bytes).
void run_layer(const csa2_layer_args *a, const LayerSizes &z, void *ws, size_t ws_bytes, void *stream) {
    hipStream_t s = (hipStream_t)stream;
    csa2::Carve c(ws, ws_bytes);
    if (a->mode != CSA2_REUSE) {
        const int BQ = a->B * a->Q;
        float *scores = a->scores ? a->scores : c.take<float>((size_t)BQ * z.n);
        auto *stats = c.take<csa2::TileStat>((size_t)BQ * z.sel.ntiles);
        auto *sumwq = c.take<double>((size_t)BQ);
        const void *qI = decode_queries(a->qI, a->idx_dt, a->B, a->Q, a->HI, a->dI, c, s);
        const int dt = kernel_idx_dt(a->idx_dt);
        void *selws = c.base + c.used;
        c.used += z.selws;
        const int32_t *cand = a->mode == CSA2_REINDEX ? a->pool : nullptr;
        csa2::launch_index_score(qI, dt, a->w, a->kI, a->B, a->Q, a->HI, a->dI, a->N, a->q_pos, a->m,
                                 cand, cand ? a->P : 0, scores, stats, sumwq, s);
        const csa2::RescoreArgs rs{qI, dt, a->w, a->kI, a->Q, a->HI, a->dI, a->N, sumwq};
        // the top-k's final pick and compaction run in the attention kernel when both sides allow
        const bool fuse = csa2::sel_handoff_supported(z.sel) && csa2::attn_handoff_supported(z.att, z.sel);
        csa2::SelHandoff h{};
        csa2::sel_run(z.sel, scores, cand, stats, &rs, a->idx, a->count,
                      a->mode == CSA2_FULL && a->P > 0 ? a->pool : nullptr, selws, z.selws, s, fuse ? &h : nullptr);
        if (fuse) {
            void *attws = c.base + c.used;
            csa2::attn_run(z.att, a->q, a->kv, a->idx, a->scale, a->out, a->lse, attws, z.attws, s, &h);
            return;
        }
    }
    void *attws = c.base + c.used;
    csa2::attn_run(z.att, a->q, a->kv, a->idx, a->scale, a->out, a->lse, attws, z.attws, s);
}

// ------------------------------------------------- allocation-free layer
// Scratch of csa2_layer_noalloc: a file-scope device array, one copy per GPU
// that the library runs on, held until the process ends.  Host code never
// passes the array's name to a kernel (on the host it is only a stand-in):
// its device address is taken once per device with hipGetSymbolAddress, with
// that device current, and kept here.
constexpr size_t NOALLOC_SCRATCH_BYTES = CSA2_NOALLOC_SCRATCH_BYTES;
constexpr int NOALLOC_MAX_DEVICES = 64;
}  // namespace
static __device__ __attribute__((aligned(256))) uint8_t scratch[NOALLOC_SCRATCH_BYTES];
namespace {
std::mutex g_scratch_mu;
void *g_scratch_dev[NOALLOC_MAX_DEVICES];

void *scratch_ptr() {
    int dev = 0;
    CSA2_HIP(hipGetDevice(&dev));
    if (dev < 0 || dev >= NOALLOC_MAX_DEVICES) throw Error(CSA2_EUNSUPPORTED, "device ordinal beyond 63");
    std::lock_guard<std::mutex> lock(g_scratch_mu);
    if (!g_scratch_dev[dev]) {
        void *p = nullptr;
        CSA2_HIP(hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)));
        if (!p || (reinterpret_cast<uintptr_t>(p) & 255u)) throw Error(CSA2_EINTERNAL, "scratch address unusable");
        g_scratch_dev[dev] = p;
    }
    return g_scratch_dev[dev];
}

}  // namespace

extern "C" {

const char *csa2_last_error(void) { return g_last_error.c_str(); }
const char *csa2_version(void) { return "csa2-mi355x 0.1 (gfx950)"; }

size_t csa2_compress_workspace_size(int dt, int64_t n_out, int32_t D, int32_t m, int32_t halo) {
    if (n_out < 1 || D < 1 || m < 1) return 0;
    return csa2::compress_workspace(dt, n_out, D, m, halo);
}

int csa2_compress(const void *x, int dt, int64_t n_out, int32_t D, int32_t m, int32_t halo, const void *wz,
                  const float *bias, void *out, void *ws, size_t ws_bytes, void *stream) {
    return guarded([&] {
        need_plain_dt(dt, "dtype");
        if (n_out < 1 || D < 1 || m < 1 || m > 16 || (halo != 0 && halo != 1))
            throw Error(CSA2_EINVAL, "need n_out >= 1, D >= 1, 1 <= m <= 16, halo in {0,1}");
        if (D % 16) throw Error(CSA2_EINVAL, "D must be a multiple of 16");
        need_ptr(x, "x");
        need_ptr(wz, "wz");
        need_ptr(bias, "bias");
        need_ptr(out, "out");
        need_ws(ws, ws_bytes, csa2::compress_workspace(dt, n_out, D, m, halo));
        csa2::compress_run(x, dt, n_out, D, m, halo, wz, bias, out, ws, ws_bytes, (hipStream_t)stream);
    });
}

size_t csa2_index_score_workspace_size(int dt, int32_t B, int32_t Q, int32_t HI, int32_t dI, int64_t N, int32_t P) {
    if (B < 1 || Q < 1 || HI < 1 || dI < 1) return 0;
    return index_ws(dt, B, Q, HI, dI, P > 0 ? P : N);
}

int csa2_index_score(const void *qI, const float *w, const void *kI, int dt, int32_t B, int32_t Q, int32_t HI,
                     int32_t dI, int64_t N, const int64_t *q_pos, int32_t m, const int32_t *cand, int32_t P,
                     float *scores, float *err, void *ws, size_t ws_bytes, void *stream) {
    return guarded([&] {
        check_index_args(dt, B, Q, HI, dI, N, P);
        need_ptr(qI, "qI");
        need_ptr(w, "w");
        need_ptr(kI, "kI");
        need_ptr(scores, "scores");
        opt_ptr(err, "err");
        opt_ptr(q_pos, "q_pos");
        opt_ptr(cand, "cand");
        if (cand && P < 1) throw Error(CSA2_EINVAL, "cand needs P >= 1");
        if (q_pos && m < 1) throw Error(CSA2_EINVAL, "m must be >= 1 with q_pos");
        if (dt == CSA2_FP4QK && (reinterpret_cast<uintptr_t>(qI) & 3))
            throw Error(CSA2_EINVAL, "FP4 query rows must be 4-byte aligned");
        const int64_t n = cand ? P : N;
        need_ws(ws, ws_bytes, index_ws(dt, B, Q, HI, dI, n));
        hipStream_t s = (hipStream_t)stream;
        csa2::Carve c(ws, ws_bytes);
        const int ntiles = (int)((n + csa2::TILE - 1) / csa2::TILE);
        auto *stats = c.take<csa2::TileStat>((size_t)B * Q * ntiles);
        const void *qk = decode_queries(qI, dt, B, Q, HI, dI, c, s);
        const int kdt = kernel_idx_dt(dt);
        csa2::launch_index_score(qk, kdt, w, kI, B, Q, HI, dI, N, q_pos, m, cand, cand ? P : 0, scores, stats, nullptr,
                                 s);
        if (err) csa2::launch_err_bound(qk, kdt, w, B * Q, HI, dI, stats, ntiles, err, nullptr, s);
    });
}

size_t csa2_topk_workspace_size(int32_t B, int32_t Q, int64_t n, int32_t k) {
    if (B < 1 || Q < 1 || n < 1 || k < 1) return 0;
    return csa2::sel_workspace(csa2::sel_plan(B * Q, n, k, 0, false), true);
}

int csa2_topk(const float *scores, int32_t B, int32_t Q, int64_t n, const int32_t *cand, int32_t k, int32_t *idx,
              int32_t *count, void *ws, size_t ws_bytes, void *stream) {
    return guarded([&] {
        if (B < 1 || Q < 1 || n < 1 || k < 1) throw Error(CSA2_EINVAL, "B, Q, n and k must be >= 1");
        if (n > INT32_MAX) throw Error(CSA2_EINVAL, "n must fit int32");
        check_queries(B, Q);
        need_ptr(scores, "scores");
        need_ptr(idx, "idx");
        opt_ptr(cand, "cand");
        opt_ptr(count, "count");
        const csa2::SelPlan p = csa2::sel_plan(B * Q, n, k, 0, false);
        need_ws(ws, ws_bytes, csa2::sel_workspace(p, true));
        csa2::sel_run(p, scores, cand, nullptr, nullptr, idx, count, nullptr, ws, ws_bytes,
                      (hipStream_t)stream);
    });
}

size_t csa2_sparse_attn_workspace_size(int q_dt, int kv_dt, int32_t B, int32_t Q, int32_t H, int32_t D, int32_t k) {
    if (B < 1 || Q < 1 || H < 1 || D < 1 || k < 1) return 0;
    return csa2::attn_workspace(csa2::attn_plan(q_dt, kv_dt, B, Q, H, D, 1, k));
}

int csa2_sparse_attn(const void *q, const void *kv, int q_dt, int kv_dt, int32_t B, int32_t Q, int32_t H, int32_t D,
                     int64_t N, const int32_t *idx, int32_t k, float scale, void *out, float *lse, void *ws,
                     size_t ws_bytes, void *stream) {
    return guarded([&] {
        if (B < 1 || Q < 1 || H < 1 || D < 1 || N < 1 || k < 1)
            throw Error(CSA2_EINVAL, "B, Q, H, D, N and k must be >= 1");
        check_queries(B, Q);
        need_plain_dt(q_dt, "q dtype");
        if (kv_dt != CSA2_F32 && kv_dt != CSA2_BF16 && kv_dt != CSA2_FP4) throw Error(CSA2_EINVAL, "unknown kv format");
        if (kv_dt == CSA2_FP4 && (D % 16 || q_dt != CSA2_BF16))
            throw Error(CSA2_EINVAL, "FP4 kv needs D % 16 == 0 and bf16 queries");
        if (kv_dt == CSA2_BF16 && D % 8) throw Error(CSA2_EINVAL, "bf16 kv rows need D % 8 == 0");
        need_ptr(q, "q");
        need_ptr(kv, "kv");
        need_ptr(idx, "idx");
        need_ptr(out, "out");
        opt_ptr(lse, "lse");
        const csa2::AttnPlan p = csa2::attn_plan(q_dt, kv_dt, B, Q, H, D, N, k);
        if (!csa2::attn_supported(p))
            throw Error(CSA2_EUNSUPPORTED, "no attention kernel for this shape (vector path needs D + k <= 16384)");
        need_ws(ws, ws_bytes, csa2::attn_workspace(p));
        csa2::attn_run(p, q, kv, idx, scale, out, lse, ws, ws_bytes, (hipStream_t)stream);
    });
}

namespace {
struct SwaSizes {
    size_t attn, idx, lse, total;
};
SwaSizes swa_sizes(int q_dt, int kv_dt, int32_t B, int32_t Q, int32_t H, int32_t D, int32_t W) {
    SwaSizes z{};
    const csa2::AttnPlan p = csa2::attn_plan(q_dt, kv_dt, B, Q, H, D, 1, W);
    csa2::Carve c(nullptr, 0);
    c.take<int32_t>((size_t)B * Q * W);
    c.take<float>((size_t)B * Q * H);
    c.take<uint8_t>((size_t)B * Q * H * D * (q_dt == CSA2_F32 ? 4 : 2));
    z.attn = csa2::attn_workspace(p);
    c.take<uint8_t>(z.attn);
    z.total = c.used;
    return z;
}
}  // namespace

size_t csa2_swa_attn_workspace_size(int q_dt, int kv_dt, int32_t B, int32_t Q, int32_t H, int32_t D, int32_t W) {
    if (B < 1 || Q < 1 || H < 1 || D < 1 || W < 1) return 0;
    return swa_sizes(q_dt, kv_dt, B, Q, H, D, W).total;
}

int csa2_swa_attn(const void *q, const void *swa_kv, int q_dt, int kv_dt, int32_t B, int32_t Q, int32_t H, int32_t D,
                  int64_t T, const int64_t *q_pos, int32_t W, float scale, const void *csa_out, const float *csa_lse,
                  void *out, float *lse, void *ws, size_t ws_bytes, void *stream) {
    return guarded([&] {
        if (B < 1 || Q < 1 || H < 1 || D < 1 || T < 1 || W < 1)
            throw Error(CSA2_EINVAL, "B, Q, H, D, T and W must be >= 1");
        check_queries(B, Q);
        need_plain_dt(q_dt, "q dtype");
        if (kv_dt != CSA2_F32 && kv_dt != CSA2_BF16 && kv_dt != CSA2_FP4) throw Error(CSA2_EINVAL, "unknown kv format");
        if (kv_dt == CSA2_FP4 && (D % 16 || q_dt != CSA2_BF16))
            throw Error(CSA2_EINVAL, "FP4 kv needs D % 16 == 0 and bf16 queries");
        if (kv_dt == CSA2_BF16 && D % 8) throw Error(CSA2_EINVAL, "bf16 kv rows need D % 8 == 0");
        need_ptr(q, "q");
        need_ptr(swa_kv, "swa_kv");
        need_ptr(q_pos, "q_pos");
        need_ptr(out, "out");
        opt_ptr(lse, "lse");
        if ((csa_out == nullptr) != (csa_lse == nullptr))
            throw Error(CSA2_EINVAL, "csa_out and csa_lse are given together or not at all");
        if (csa_out) {
            opt_ptr(csa_out, "csa_out");
            opt_ptr(csa_lse, "csa_lse");
            if (D % 8) throw Error(CSA2_EINVAL, "the merge needs D % 8 == 0");
        }
        const csa2::AttnPlan p = csa2::attn_plan(q_dt, kv_dt, B, Q, H, D, T, W);
        if (!csa2::attn_supported(p))
            throw Error(CSA2_EUNSUPPORTED, "no attention kernel for this shape (vector path needs D + W <= 16384)");
        const SwaSizes z = swa_sizes(q_dt, kv_dt, B, Q, H, D, W);
        need_ws(ws, ws_bytes, z.total);
        hipStream_t s = (hipStream_t)stream;
        csa2::Carve c(ws, ws_bytes);
        int32_t *idx = c.take<int32_t>((size_t)B * Q * W);
        float *lse_w = c.take<float>((size_t)B * Q * H);
        void *out_w = c.take<uint8_t>((size_t)B * Q * H * D * (q_dt == CSA2_F32 ? 4 : 2));
        void *aws = c.take<uint8_t>(z.attn);
        const int64_t BQ = (int64_t)B * Q;
        csa2::launch_window_idx(q_pos, BQ, W, T, idx, s);
        if (!csa_out) {
            csa2::attn_run(p, q, swa_kv, idx, scale, out, lse, aws, z.attn, s);
            return;
        }
        // the window branch goes to the workspace (out may be csa_out), then
        // the two are merged into out
        csa2::attn_run(p, q, swa_kv, idx, scale, out_w, lse_w, aws, z.attn, s);
        csa2::launch_merge_attn(q_dt, csa_out, csa_lse, out_w, lse_w, BQ * H, D, out, lse, s);
    });
}

int csa2_merge_attn(const void *o_a, const float *lse_a, const void *o_b, const float *lse_b, int dt, int64_t R,
                    int32_t D, void *out, float *lse, void *stream) {
    return guarded([&] {
        if (R < 1 || D < 8 || D % 8) throw Error(CSA2_EINVAL, "R >= 1 and D a positive multiple of 8 are needed");
        need_plain_dt(dt, "dtype");
        need_ptr(o_a, "o_a");
        need_ptr(lse_a, "lse_a");
        need_ptr(o_b, "o_b");
        need_ptr(lse_b, "lse_b");
        need_ptr(out, "out");
        opt_ptr(lse, "lse");
        csa2::launch_merge_attn(dt, o_a, lse_a, o_b, lse_b, R, D, out, lse, (hipStream_t)stream);
    });
}

int csa2_quantize_fp4(const void *x, int dt, int64_t n, int32_t D, void *cache, const int64_t *dst_row,
                      void *stream) {
    return guarded([&] {
        if (n < 1 || D < 16 || D % 16) throw Error(CSA2_EINVAL, "n >= 1 and D a positive multiple of 16 are needed");
        need_plain_dt(dt, "x dtype");
        need_ptr(x, "x");
        if (!cache) throw Error(CSA2_EINVAL, "cache is NULL");  // rows are byte-addressed: no alignment needed
        if (dst_row && (reinterpret_cast<uintptr_t>(dst_row) & 7u)) throw Error(CSA2_EINVAL, "dst_row is not aligned");
        csa2::launch_quantize_fp4(x, dt, n, D, static_cast<uint8_t *>(cache), dst_row, (hipStream_t)stream);
    });
}

size_t csa2_layer_workspace_size(const csa2_layer_args *a) {
    if (!a || a->B < 1 || a->Q < 1 || a->k < 1 || a->H < 1 || a->D < 1) return 0;
    if ((int64_t)a->B * a->Q > MAX_QUERIES) return 0;
    return layer_sizes(a).total;
}

size_t csa2_workspace_size(const csa2_layer_args *a) { return csa2_layer_workspace_size(a); }

int csa2_layer(const csa2_layer_args *a, void *ws, size_t ws_bytes, void *stream) {
    return guarded([&] {
        check_layer(a);
        const LayerSizes z = layer_sizes(a);
        need_ws(ws, ws_bytes, z.total);
        run_layer(a, z, ws, ws_bytes, stream);
    });
}

int csa2_layer_noalloc(const csa2_layer_args *a, void *stream) {
    return guarded([&] {
        check_layer(a);
        const LayerSizes z = layer_sizes(a);
        if (z.total > NOALLOC_SCRATCH_BYTES)
            throw Error(CSA2_EUNSUPPORTED, "this layer needs " + std::to_string(z.total) +
                                               " bytes of scratch; the allocation-free entry point has " +
                                               std::to_string(NOALLOC_SCRATCH_BYTES));
        run_layer(a, z, scratch_ptr(), NOALLOC_SCRATCH_BYTES, stream);
    });
}

}  // extern "C"
