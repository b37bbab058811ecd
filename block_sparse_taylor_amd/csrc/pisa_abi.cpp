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
    if (p->cov_bias != 0 && p->cov_bias != 1) return PISA_ERR_PARAM;
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

// The statistics a call reads: kbar, vsum, hsum always (the fp32 attention
// and the backward read them, the router kbar), qbar for the router, and the
// second-order pair when the term is on.
pisa_status_t check_stats(const pisa_stats_t* st, int second_order, bool need_qbar) {
    if (!st) return PISA_ERR_NULL;
    PISA_TRY(check_ptr(st->kbar));
    PISA_TRY(check_ptr(st->vsum));
    PISA_TRY(check_ptr(st->hsum));
    if (need_qbar) PISA_TRY(check_ptr(st->qbar));
    if (second_order) {
        PISA_TRY(check_ptr(st->ksig2));
        PISA_TRY(check_ptr(st->q2bar));
    } else {
        if (st->ksig2 && !aligned16(st->ksig2)) return PISA_ERR_ALIGN;
        if (st->q2bar && !aligned16(st->q2bar)) return PISA_ERR_ALIGN;
    }
    return PISA_OK;
}

pisa_status_t check_operands(const Geom& g, int dtype, const void* operands, size_t bytes) {
    PISA_TRY(check_ptr(operands));
    if (bytes < operand_layout(g, dtype).total) return PISA_ERR_WORKSPACE;
    return PISA_OK;
}

// [a, a + na) and [b, b + nb) share a byte
bool overlap(const void* a, size_t na, const void* b, size_t nb) {
    const uintptr_t x = reinterpret_cast<uintptr_t>(a), y = reinterpret_cast<uintptr_t>(b);
    return a && b && x < y + nb && y < x + na;
}

size_t tensor_bytes(const Geom& g, int dtype) {
    return (size_t)g.BH * g.T * g.D * (dtype == PISA_BF16 ? 2 : 4);
}

pisa_status_t from_hip(hipError_t e) { return e == hipSuccess ? PISA_OK : PISA_ERR_HIP; }

// bytes of a [B,H,T,2] fp32 row-statistics array
size_t row_stats_bytes(const Geom& g) { return (size_t)g.BH * (size_t)g.T * 2 * sizeof(float); }

pisa_status_t attn_common(const pisa_shape_t* shape, const pisa_params_t* params, const void* q,
                          const void* k, const void* v, const pisa_stats_t* stats, const void* operands,
                          size_t operands_bytes, const int32_t* idx, const float* wgate, void* o,
                          const float* row_stats, Geom* g, bool need_operands) {
    PISA_TRY(check_shape(shape, g));
    PISA_TRY(check_params(params, *g));
    PISA_TRY(check_ptr(q));
    PISA_TRY(check_ptr(k));
    PISA_TRY(check_ptr(v));
    PISA_TRY(check_ptr(o));
    PISA_TRY(check_stats(stats, 0, false));
    if (need_operands) PISA_TRY(check_operands(*g, shape->dtype, operands, operands_bytes));
    if (params->topk > 0) PISA_TRY(check_ptr(idx));
    if (params->second_order) PISA_TRY(check_ptr(wgate));
    const size_t tb = tensor_bytes(*g, shape->dtype);
    if (overlap(o, tb, q, tb) || overlap(o, tb, k, tb) || overlap(o, tb, v, tb)) return PISA_ERR_PARAM;
    if (row_stats) {   // an optional output: shares no byte with o or the inputs
        PISA_TRY(check_ptr(row_stats));
        const size_t rb = row_stats_bytes(*g);
        for (const void* t : {static_cast<const void*>(q), k, v, static_cast<const void*>(o)})
            if (overlap(row_stats, rb, t, tb)) return PISA_ERR_PARAM;
    }
    return PISA_OK;
}

}  // namespace

namespace pisa {

OperandLayout operand_layout(const Geom& g, int dtype) {
    const size_t e = dtype == PISA_BF16 ? 2 : 4;
    const bool bf = dtype == PISA_BF16;
    const size_t BH = (size_t)g.BH, N = (size_t)g.N, D = (size_t)g.D;
    size_t sz[PISA_OPERAND_COUNT];
    sz[PISA_OPERAND_KBAR_C] = BH * N * D * e;
    sz[PISA_OPERAND_VBAR_C] = BH * N * D * e;
    sz[PISA_OPERAND_KBAR_R] = BH * ((N + 15) / 16) * 16 * D * 4;
    sz[PISA_OPERAND_KSIG2_R] = sz[PISA_OPERAND_KBAR_R];
    sz[PISA_OPERAND_KPACK] = bf ? BH * N * 64 * D * 2 : 0;
    sz[PISA_OPERAND_KBPACK] = bf ? BH * ((N + 63) / 64) * 64 * D * 2 : 0;
    sz[PISA_OPERAND_HPACK] = bf ? BH * 2 * D * D * 2 : 0;
    sz[PISA_OPERAND_KNORM] = BH * ((N + 15) / 16) * 16 * 4;
    OperandLayout L{};
    size_t at = 0;
    for (int i = 0; i < PISA_OPERAND_COUNT; ++i) {
        L.off[i] = at;
        L.bytes[i] = sz[i];
        at += (sz[i] + 255) / 256 * 256;
    }
    L.total = at;
    return L;
}

StatsView stats_view(const Geom& g, int dtype, const pisa_stats_t* st, const void* operands) {
    StatsView v{};
    v.qbar = st->qbar;
    v.q2bar = st->q2bar;
    v.kbar = st->kbar;
    v.vsum = st->vsum;
    v.ksig2 = st->ksig2;
    v.hsum = st->hsum;
    v.hnorm = st->hnorm;
    if (operands) {
        const OperandLayout L = operand_layout(g, dtype);
        char* b = static_cast<char*>(const_cast<void*>(operands));
        auto at = [&](int i) -> void* { return L.bytes[i] ? b + L.off[i] : nullptr; };
        v.kbar_c = at(PISA_OPERAND_KBAR_C);
        v.vbar_c = at(PISA_OPERAND_VBAR_C);
        v.kbar_r = static_cast<bf16_t*>(at(PISA_OPERAND_KBAR_R));
        v.ksig2_r = static_cast<bf16_t*>(at(PISA_OPERAND_KSIG2_R));
        v.knorm = static_cast<float*>(at(PISA_OPERAND_KNORM));
        v.kpack = at(PISA_OPERAND_KPACK);
        v.kbpack = at(PISA_OPERAND_KBPACK);
        v.hpack = at(PISA_OPERAND_HPACK);
    }
    return v;
}

}  // namespace pisa

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

size_t pisa_operands_bytes(const pisa_shape_t* shape) {
    Geom g;
    if (check_shape(shape, &g) != PISA_OK) return 0;
    return operand_layout(g, shape->dtype).total;
}

pisa_status_t pisa_operands_offsets(const pisa_shape_t* shape, int64_t* offsets) {
    Geom g;
    PISA_TRY(check_shape(shape, &g));
    if (!offsets) return PISA_ERR_NULL;
    const OperandLayout L = operand_layout(g, shape->dtype);
    for (int i = 0; i < PISA_OPERAND_COUNT; ++i) offsets[i] = (int64_t)L.off[i];
    return PISA_OK;
}

pisa_status_t pisa_block_stats(const pisa_shape_t* shape, const pisa_params_t* params, const void* q,
                               const void* k, const void* v, const pisa_stats_t* out, void* operands,
                               size_t operands_bytes, void* workspace, size_t workspace_bytes, void* stream) {
    Geom g;
    PISA_TRY(check_shape(shape, &g));
    PISA_TRY(check_params(params, g));
    PISA_TRY(check_ptr(q));
    PISA_TRY(check_ptr(k));
    PISA_TRY(check_ptr(v));
    PISA_TRY(check_stats(out, params->second_order, true));
    if (params->cov_bias) PISA_TRY(check_ptr(out->hnorm));
    PISA_TRY(check_operands(g, shape->dtype, operands, operands_bytes));
    PISA_TRY(check_ptr(workspace));
    if (workspace_bytes < stats_workspace_bytes_for(g, params->cov_bias)) return PISA_ERR_WORKSPACE;
    const size_t tb = tensor_bytes(g, shape->dtype), ob = operand_layout(g, shape->dtype).total;
    for (const void* in : {q, k, v})
        if (overlap(operands, ob, in, tb) || overlap(workspace, workspace_bytes, in, tb)) return PISA_ERR_PARAM;
    if (overlap(operands, ob, workspace, workspace_bytes)) return PISA_ERR_PARAM;
    const StatsView sv = stats_view(g, shape->dtype, out, operands);
    return from_hip(launch_block_stats(g, shape->dtype, params->second_order, params->cov_bias, q, k, v, &sv,
                                       workspace, static_cast<hipStream_t>(stream)));
}

pisa_status_t pisa_block_stats_noalloc(const pisa_shape_t* shape, const pisa_params_t* params, const void* q,
                                       const void* k, const void* v, const pisa_stats_t* out, void* operands,
                                       size_t operands_bytes, void* stream) {
    Geom g;
    PISA_TRY(check_shape(shape, &g));
    PISA_TRY(check_params(params, g));
    PISA_TRY(check_ptr(q));
    PISA_TRY(check_ptr(k));
    PISA_TRY(check_ptr(v));
    PISA_TRY(check_stats(out, params->second_order, true));
    if (params->cov_bias) PISA_TRY(check_ptr(out->hnorm));
    PISA_TRY(check_operands(g, shape->dtype, operands, operands_bytes));
    if (stats_workspace_bytes_for(g, params->cov_bias) > PISA_STATS_SCRATCH_BYTES) return PISA_ERR_WORKSPACE;
    const size_t tb = tensor_bytes(g, shape->dtype), ob = operand_layout(g, shape->dtype).total;
    for (const void* in : {q, k, v})
        if (overlap(operands, ob, in, tb)) return PISA_ERR_PARAM;
    void* ws = nullptr;
    PISA_TRY(from_hip(stats_scratch(&ws)));
    const StatsView sv = stats_view(g, shape->dtype, out, operands);
    return from_hip(launch_block_stats(g, shape->dtype, params->second_order, params->cov_bias, q, k, v, &sv, ws,
                                       static_cast<hipStream_t>(stream)));
}

pisa_status_t pisa_prepare_operands(const pisa_shape_t* shape, const pisa_params_t* params, const void* k,
                                    const pisa_stats_t* stats, void* operands, size_t operands_bytes,
                                    void* stream) {
    Geom g;
    PISA_TRY(check_shape(shape, &g));
    PISA_TRY(check_params(params, g));
    if (shape->dtype == PISA_BF16) PISA_TRY(check_ptr(k));
    PISA_TRY(check_stats(stats, params->second_order, false));
    PISA_TRY(check_operands(g, shape->dtype, operands, operands_bytes));
    const size_t ob = operand_layout(g, shape->dtype).total;
    if (overlap(operands, ob, k, tensor_bytes(g, shape->dtype))) return PISA_ERR_PARAM;
    const StatsView sv = stats_view(g, shape->dtype, stats, operands);
    return from_hip(launch_prepare_operands(g, shape->dtype, params->second_order, k, &sv,
                                            static_cast<hipStream_t>(stream)));
}

pisa_status_t pisa_route_topk(const pisa_shape_t* shape, const pisa_params_t* params,
                              const pisa_stats_t* stats, const void* operands, size_t operands_bytes,
                              int32_t* idx, float* wgate, void* stream) {
    Geom g;
    PISA_TRY(check_shape(shape, &g));
    PISA_TRY(check_params(params, g));
    PISA_TRY(check_stats(stats, params->second_order, true));
    if (params->cov_bias) PISA_TRY(check_ptr(stats->hnorm));
    PISA_TRY(check_operands(g, shape->dtype, operands, operands_bytes));
    if (params->second_order) PISA_TRY(check_ptr(wgate));
    if (params->topk > 0) PISA_TRY(check_ptr(idx));
    const pisa_params_t pr = resolved(params, g);
    const StatsView sv = stats_view(g, shape->dtype, stats, operands);
    return from_hip(launch_route_topk(g, &pr, &sv, idx, wgate, static_cast<hipStream_t>(stream)));
}

pisa_status_t pisa_attn_fwd(const pisa_shape_t* shape, const pisa_params_t* params, const void* q,
                            const void* k, const void* v, const pisa_stats_t* stats, const void* operands,
                            size_t operands_bytes, const int32_t* idx, const float* wgate, void* o,
                            float* row_stats, void* stream) {
    Geom g;
    const bool bf = shape && shape->dtype == PISA_BF16;
    PISA_TRY(attn_common(shape, params, q, k, v, stats, operands, operands_bytes, idx, wgate, o, row_stats, &g, bf));
    hipStream_t s = static_cast<hipStream_t>(stream);
    const pisa_params_t pr = resolved(params, g);
    const StatsView sv = stats_view(g, shape->dtype, stats, bf ? operands : nullptr);
    if (bf) return from_hip(launch_attn_fwd_mfma(g, &pr, q, k, v, &sv, idx, wgate, o, row_stats, s));
    return from_hip(launch_attn_fwd_f32(g, &pr, q, k, v, &sv, idx, wgate, o, row_stats, s));
}

pisa_status_t pisa_attn_fwd_valu(const pisa_shape_t* shape, const pisa_params_t* params,
                                 const void* q, const void* k, const void* v,
                                 const pisa_stats_t* stats, const void* operands, size_t operands_bytes,
                                 const int32_t* idx, const float* wgate, void* o, float* row_stats,
                                 void* stream) {
    Geom g;
    PISA_TRY(attn_common(shape, params, q, k, v, stats, operands, operands_bytes, idx, wgate, o, row_stats, &g,
                         false));
    const pisa_params_t pr = resolved(params, g);
    const StatsView sv = stats_view(g, shape->dtype, stats, nullptr);
    return from_hip(launch_attn_fwd_valu(g, shape->dtype, &pr, q, k, v, &sv, idx, wgate, o, row_stats,
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
                            const pisa_stats_t* stats, const int32_t* idx, const float* wgate,
                            const float* row_stats, void* dq, void* dk, void* dv, void* workspace,
                            size_t workspace_bytes, void* stream) {
    Geom g;
    PISA_TRY(check_shape(shape, &g));
    PISA_TRY(check_params(params, g));
    const void* ptrs[9] = {q, k, v, o, dout, dq, dk, dv, workspace};
    for (const void* ptr : ptrs) PISA_TRY(check_ptr(ptr));
    PISA_TRY(check_stats(stats, params->second_order, false));
    if (params->topk > 0) PISA_TRY(check_ptr(idx));
    if (params->second_order) PISA_TRY(check_ptr(wgate));
    if (row_stats) PISA_TRY(check_ptr(row_stats));
    if (params->phase_mask != 0) return PISA_ERR_UNSUPPORTED;
    if (workspace_bytes < attn_bwd_workspace_bytes(g, shape->dtype)) return PISA_ERR_WORKSPACE;
    // no output may share a byte with another output, an input or the workspace
    const size_t tb = tensor_bytes(g, shape->dtype);
    const void* outs[3] = {dq, dk, dv};
    const void* ins[5] = {q, k, v, o, dout};
    for (int a = 0; a < 3; ++a) {
        for (int b = a + 1; b < 3; ++b)
            if (overlap(outs[a], tb, outs[b], tb)) return PISA_ERR_PARAM;
        for (const void* in : ins)
            if (overlap(outs[a], tb, in, tb)) return PISA_ERR_PARAM;
        if (overlap(outs[a], tb, workspace, workspace_bytes)) return PISA_ERR_PARAM;
        if (row_stats && overlap(outs[a], tb, row_stats, row_stats_bytes(g))) return PISA_ERR_PARAM;
    }
    if (row_stats && overlap(workspace, workspace_bytes, row_stats, row_stats_bytes(g))) return PISA_ERR_PARAM;
    const pisa_params_t pr = resolved(params, g);
    const StatsView sv = stats_view(g, shape->dtype, stats, nullptr);
    return from_hip(launch_attn_bwd(g, shape->dtype, &pr, q, k, v, o, dout, &sv, idx, wgate, row_stats, dq, dk,
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
