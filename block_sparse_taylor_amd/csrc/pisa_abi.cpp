// C ABI of libpisa: host-side argument validation and kernel dispatch.
// Every check runs before the first HIP call, so invalid requests return a
// status without touching the device (and can be tested on a GPU-less host).
#include <math.h>
#include <stdint.h>

#include "common.h"

using namespace pisa;

namespace {

constexpr int64_t kMaxSeq = 524288;   // N <= 8192 blocks
constexpr int64_t kMaxBH = 65535;     // grid y dimension

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

pisa_status_t check_shape(const pisa_shape_t* s, Geom* g) {
    if (!s) return PISA_ERR_NULL;
    if (s->dtype != PISA_F32 && s->dtype != PISA_BF16) return PISA_ERR_DTYPE;
    if (s->batch < 1 || s->heads < 1 || s->seq_len < 1 || s->seq_len > kMaxSeq) return PISA_ERR_SHAPE;
    if (s->batch > kMaxBH || s->heads > kMaxBH || s->batch * s->heads > kMaxBH) return PISA_ERR_SHAPE;
    if (s->head_dim != 64 && s->head_dim != 128) return PISA_ERR_SHAPE;
    if (s->block_size != kBlock) return PISA_ERR_PARAM;
    if (!isfinite(s->scale)) return PISA_ERR_PARAM;
    if (g) {
        g->BH = s->batch * s->heads;
        g->T = (int)s->seq_len;
        g->D = (int)s->head_dim;
        g->N = (int)((s->seq_len + kBlock - 1) / kBlock);
        g->scale64 = s->scale > 0.f ? (double)s->scale : 1.0 / sqrt((double)s->head_dim);
        g->scale = (float)g->scale64;
    }
    return PISA_OK;
}

pisa_status_t check_params(const pisa_params_t* p, const Geom& g) {
    if (!p) return PISA_ERR_NULL;
    if (p->topk < 0 || p->topk > g.N) return PISA_ERR_PARAM;
    if (p->band < 0) return PISA_ERR_PARAM;
    if (p->second_order != 0 && p->second_order != 1) return PISA_ERR_PARAM;
    if (p->first_order != 0 && p->first_order != 1) return PISA_ERR_PARAM;
    if (p->phase_mask < 0 || p->phase_mask > 7) return PISA_ERR_PARAM;
    if (p->n_sink < 0 || p->n_sink > g.N) return PISA_ERR_PARAM;
    return PISA_OK;
}

// The parameters the kernels see: a band of N or more already makes every
// block exact, so it is clamped to N (int arithmetic on i +- band stays in
// range for any band the caller passes).
pisa_params_t resolved(const pisa_params_t* p, const Geom& g) {
    pisa_params_t r = *p;
    if (r.band > g.N) r.band = g.N;
    return r;
}

pisa_status_t check_ptr(const void* p) {
    if (!p) return PISA_ERR_NULL;
    return aligned16(p) ? PISA_OK : PISA_ERR_ALIGN;
}

#define PISA_TRY(expr)                        \
    do {                                      \
        pisa_status_t st_ = (expr);           \
        if (st_ != PISA_OK) return st_;       \
    } while (0)

pisa_status_t check_stats(const pisa_stats_t* st, int second_order, bool need_c, bool need_kpack) {
    if (!st) return PISA_ERR_NULL;
    PISA_TRY(check_ptr(st->kbar));
    PISA_TRY(check_ptr(st->vsum));
    PISA_TRY(check_ptr(st->hsum));
    if (need_c) {
        PISA_TRY(check_ptr(st->kbar_c));
        PISA_TRY(check_ptr(st->vbar_c));
    }
    if (need_kpack) {
        PISA_TRY(check_ptr(st->kpack));
        PISA_TRY(check_ptr(st->hpack));
        PISA_TRY(check_ptr(st->kbpack));
    }
    if (second_order) PISA_TRY(check_ptr(st->ksig2));
    else if (st->ksig2 && !aligned16(st->ksig2)) return PISA_ERR_ALIGN;
    return PISA_OK;
}

pisa_status_t from_hip(hipError_t e) { return e == hipSuccess ? PISA_OK : PISA_ERR_HIP; }

pisa_status_t attn_common(const pisa_shape_t* shape, const pisa_params_t* params, const void* q,
                          const void* k, const void* v, const pisa_stats_t* stats,
                          const int32_t* idx, const float* wgate, void* o, Geom* g) {
    PISA_TRY(check_shape(shape, g));
    PISA_TRY(check_params(params, *g));
    PISA_TRY(check_ptr(q));
    PISA_TRY(check_ptr(k));
    PISA_TRY(check_ptr(v));
    PISA_TRY(check_ptr(o));
    PISA_TRY(check_stats(stats, 0, shape->dtype == PISA_BF16, shape->dtype == PISA_BF16));
    if (params->topk > 0) PISA_TRY(check_ptr(idx));
    if (params->second_order) PISA_TRY(check_ptr(wgate));
    if (o == q || o == k || o == v) return PISA_ERR_PARAM;
    return PISA_OK;
}

}  // namespace

extern "C" {

int pisa_abi_version(void) { return PISA_ABI_VERSION; }

const char* pisa_status_str(pisa_status_t s) {
    switch (s) {
        case PISA_OK: return "ok";
        case PISA_ERR_NULL: return "null pointer";
        case PISA_ERR_SHAPE: return "shape out of range";
        case PISA_ERR_DTYPE: return "unknown dtype";
        case PISA_ERR_PARAM: return "parameter out of range";
        case PISA_ERR_ALIGN: return "pointer not 16-byte aligned";
        case PISA_ERR_UNSUPPORTED: return "unsupported";
        case PISA_ERR_HIP: return "HIP launch/runtime error";
        case PISA_ERR_WORKSPACE: return "workspace too small";
    }
    return "unknown status";
}

int64_t pisa_num_blocks(const pisa_shape_t* shape) {
    Geom g;
    if (check_shape(shape, &g) != PISA_OK) return -1;
    return g.N;
}

size_t pisa_stats_workspace_bytes(const pisa_shape_t* shape) {
    Geom g;
    if (check_shape(shape, &g) != PISA_OK) return 0;
    return stats_workspace_bytes(g);
}

pisa_status_t pisa_block_stats(const pisa_shape_t* shape, const pisa_params_t* params, const void* q,
                               const void* k, const void* v, const pisa_stats_t* out, void* workspace,
                               size_t workspace_bytes, void* stream) {
    Geom g;
    PISA_TRY(check_shape(shape, &g));
    PISA_TRY(check_params(params, g));
    PISA_TRY(check_ptr(q));
    PISA_TRY(check_ptr(k));
    PISA_TRY(check_ptr(v));
    PISA_TRY(check_stats(out, params->second_order, true, shape->dtype == PISA_BF16));
    PISA_TRY(check_ptr(out->qbar));
    PISA_TRY(check_ptr(out->kbar_r));
    if (params->second_order) PISA_TRY(check_ptr(out->ksig2_r));
    if (params->second_order) PISA_TRY(check_ptr(out->q2bar));
    PISA_TRY(check_ptr(workspace));
    if (workspace_bytes < stats_workspace_bytes(g)) return PISA_ERR_WORKSPACE;
    return from_hip(launch_block_stats(g, shape->dtype, params->second_order, q, k, v, out,
                                       workspace, static_cast<hipStream_t>(stream)));
}

pisa_status_t pisa_route_topk(const pisa_shape_t* shape, const pisa_params_t* params,
                              const pisa_stats_t* stats, int32_t* idx, float* wgate, void* stream) {
    Geom g;
    PISA_TRY(check_shape(shape, &g));
    PISA_TRY(check_params(params, g));
    if (!stats) return PISA_ERR_NULL;
    PISA_TRY(check_ptr(stats->qbar));
    PISA_TRY(check_ptr(stats->kbar));
    PISA_TRY(check_ptr(stats->kbar_r));
    if (params->second_order) PISA_TRY(check_ptr(stats->ksig2_r));
    if (params->second_order) {
        PISA_TRY(check_ptr(stats->q2bar));
        PISA_TRY(check_ptr(stats->ksig2));
        PISA_TRY(check_ptr(wgate));
    }
    if (params->topk > 0) PISA_TRY(check_ptr(idx));
    const pisa_params_t pr = resolved(params, g);
    return from_hip(launch_route_topk(g, &pr, stats, idx, wgate, static_cast<hipStream_t>(stream)));
}

pisa_status_t pisa_attn_fwd(const pisa_shape_t* shape, const pisa_params_t* params, const void* q,
                            const void* k, const void* v, const pisa_stats_t* stats,
                            const int32_t* idx, const float* wgate, void* o, void* stream) {
    Geom g;
    PISA_TRY(attn_common(shape, params, q, k, v, stats, idx, wgate, o, &g));
    hipStream_t s = static_cast<hipStream_t>(stream);
    const pisa_params_t pr = resolved(params, g);
    if (shape->dtype == PISA_BF16)
        return from_hip(launch_attn_fwd_mfma(g, &pr, q, k, v, stats, idx, wgate, o, s));
    return from_hip(launch_attn_fwd_valu(g, shape->dtype, &pr, q, k, v, stats, idx, wgate, o, s));
}

pisa_status_t pisa_attn_fwd_valu(const pisa_shape_t* shape, const pisa_params_t* params,
                                 const void* q, const void* k, const void* v,
                                 const pisa_stats_t* stats, const int32_t* idx, const float* wgate,
                                 void* o, void* stream) {
    Geom g;
    PISA_TRY(attn_common(shape, params, q, k, v, stats, idx, wgate, o, &g));
    const pisa_params_t pr = resolved(params, g);
    return from_hip(launch_attn_fwd_valu(g, shape->dtype, &pr, q, k, v, stats, idx, wgate, o,
                                         static_cast<hipStream_t>(stream)));
}

pisa_status_t pisa_attn_fwd_plan(const pisa_shape_t* shape, const pisa_params_t* params, int32_t* kernel,
                                 int64_t* wave_items) {
    Geom g;
    PISA_TRY(check_shape(shape, &g));
    PISA_TRY(check_params(params, g));
    const pisa_params_t pr = resolved(params, g);
    if (kernel) *kernel = attn_fwd_kernel(g, shape->dtype, &pr);
    if (wave_items) *wave_items = attn_asm_wave_items(g, &pr);
    return PISA_OK;
}

size_t pisa_attn_bwd_workspace_bytes(const pisa_shape_t* shape) {
    Geom g;
    if (check_shape(shape, &g) != PISA_OK) return 0;
    return attn_bwd_workspace_bytes(g, shape->dtype);
}

pisa_status_t pisa_attn_bwd(const pisa_shape_t* shape, const pisa_params_t* params, const void* q,
                            const void* k, const void* v, const void* o, const void* dout,
                            const pisa_stats_t* stats, const int32_t* idx, const float* wgate, void* dq,
                            void* dk, void* dv, void* workspace, size_t workspace_bytes, void* stream) {
    Geom g;
    PISA_TRY(check_shape(shape, &g));
    PISA_TRY(check_params(params, g));
    const void* ptrs[9] = {q, k, v, o, dout, dq, dk, dv, workspace};
    for (const void* ptr : ptrs) PISA_TRY(check_ptr(ptr));
    PISA_TRY(check_stats(stats, params->second_order, false, false));
    if (params->second_order) PISA_TRY(check_ptr(stats->q2bar));
    if (params->topk > 0) PISA_TRY(check_ptr(idx));
    if (params->second_order) PISA_TRY(check_ptr(wgate));
    if (params->phase_mask != 0) return PISA_ERR_UNSUPPORTED;
    if (workspace_bytes < attn_bwd_workspace_bytes(g, shape->dtype)) return PISA_ERR_WORKSPACE;
    const void* outs[3] = {dq, dk, dv};
    const void* ins[6] = {q, k, v, o, dout, workspace};
    for (int a = 0; a < 3; ++a) {
        for (int b = a + 1; b < 3; ++b)
            if (outs[a] == outs[b]) return PISA_ERR_PARAM;
        for (const void* in : ins)
            if (outs[a] == in) return PISA_ERR_PARAM;
    }
    const pisa_params_t pr = resolved(params, g);
    return from_hip(launch_attn_bwd(g, shape->dtype, &pr, q, k, v, o, dout, stats, idx, wgate, dq, dk,
                                    dv, workspace, static_cast<hipStream_t>(stream)));
}

pisa_status_t pisa_z_order(const int64_t* grid, int32_t ndim, int64_t prefix, int32_t* perm, int64_t n) {
    if (!grid || !perm) return PISA_ERR_NULL;
    if (ndim < 1 || ndim > 4 || prefix < 0) return PISA_ERR_SHAPE;
    int64_t cells = 1;
    int nb = 1;
    for (int a = 0; a < ndim; ++a) {
        if (grid[a] < 1 || grid[a] > 0x7fffffff) return PISA_ERR_SHAPE;
        cells *= grid[a];
        if (cells > 0x7fffffff) return PISA_ERR_SHAPE;
        while ((int64_t{1} << nb) < grid[a]) ++nb;
    }
    if (ndim * nb > 63 || prefix > 0x7fffffff - cells || n != prefix + cells) return PISA_ERR_SHAPE;
    z_order_host(grid, ndim, prefix, perm);
    return PISA_OK;
}

static pisa_status_t reorder_common(const pisa_shape_t* shape, const int32_t* perm, const void* src,
                                    void* dst, bool gather, void* stream) {
    Geom g;
    PISA_TRY(check_shape(shape, &g));
    PISA_TRY(check_ptr(perm));
    PISA_TRY(check_ptr(src));
    PISA_TRY(check_ptr(dst));
    const int e = shape->dtype == PISA_BF16 ? 2 : 4;
    const uint64_t bytes = (uint64_t)shape->batch * shape->heads * shape->seq_len * shape->head_dim * e;
    const uintptr_t a = reinterpret_cast<uintptr_t>(src), b = reinterpret_cast<uintptr_t>(dst);
    if (a < b + bytes && b < a + bytes) return PISA_ERR_PARAM;   // overlapping buffers
    return from_hip(launch_reorder(g, shape->batch, shape->heads, e, gather, perm, src, dst,
                                   static_cast<hipStream_t>(stream)));
}

pisa_status_t pisa_reorder_gather(const pisa_shape_t* shape, const int32_t* perm, const void* x, void* out,
                                  void* stream) {
    return reorder_common(shape, perm, x, out, true, stream);
}

pisa_status_t pisa_reorder_scatter(const pisa_shape_t* shape, const int32_t* perm, const void* o, void* y,
                                   void* stream) {
    return reorder_common(shape, perm, o, y, false, stream);
}

}  // extern "C"
