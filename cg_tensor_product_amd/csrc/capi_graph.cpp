// C ABI entry points on the graph side: the sender CSR and sender view, the CSR
// check, the schedule model's choice and the sender-stationary passes.
#include "capi_internal.hpp"

using namespace oeq::capi;

extern "C" {

oeq_status oeq_plan_schedule(const oeq_plan *p, oeq_schedule *fwd, oeq_schedule *bwd, double *move_fwd2,
                             double *move_bwd2) {
    if (!p) return fail(OEQ_ERR_INVALID_ARG, "plan is NULL");
    if (fwd) *fwd = p->sched_fwd ? OEQ_SENDER_STATIONARY : OEQ_RECEIVER_STATIONARY;
    if (bwd) *bwd = p->sched_bwd ? OEQ_SENDER_STATIONARY : OEQ_RECEIVER_STATIONARY;
    if (move_fwd2) std::memcpy(move_fwd2, p->move_fwd, sizeof p->move_fwd);
    if (move_bwd2) std::memcpy(move_bwd2, p->move_bwd, sizeof p->move_bwd);
    return OEQ_OK;
}

oeq_status oeq_csr_workspace_size(int64_t n_nodes, int64_t n_edges, size_t *bytes) {
    if (!bytes || n_nodes < 0 || n_edges < 0) return fail(OEQ_ERR_INVALID_ARG, "bad arguments");
    const hipError_t e = oeq::sender_csr_workspace(n_nodes, n_edges, bytes);
    if (e != hipSuccess) return fail(OEQ_ERR_HIP, hipGetErrorString(e));
    return OEQ_OK;
}

oeq_status oeq_sender_csr(int64_t n_nodes, int64_t n_edges, const int32_t *src, int32_t *srowptr, int32_t *sperm,
                          void *workspace, size_t workspace_bytes, void *stream) {
    if (n_nodes < 0 || n_edges < 0) return fail(OEQ_ERR_INVALID_ARG, "negative size");
    if (n_nodes >= std::numeric_limits<int32_t>::max() || n_edges >= std::numeric_limits<int32_t>::max())
        return fail(OEQ_ERR_UNSUPPORTED, "sizes must fit int32");
    if (!srowptr || (n_edges > 0 && (!src || !sperm))) return fail(OEQ_ERR_INVALID_ARG, "NULL array");
    size_t need = 0;
    oeq_status st = oeq_csr_workspace_size(n_nodes, n_edges, &need);
    if (st != OEQ_OK) return st;
    if (!workspace || workspace_bytes < need) return fail(OEQ_ERR_WORKSPACE, "workspace too small");
    if (reinterpret_cast<uintptr_t>(workspace) % kAlign)
        return fail(OEQ_ERR_WORKSPACE, "workspace must be 256-byte aligned");
    const hipError_t e = oeq::sender_csr(n_nodes, n_edges, src, srowptr, sperm, workspace,
                                         static_cast<hipStream_t>(stream));
    if (e != hipSuccess) return fail(OEQ_ERR_HIP, hipGetErrorString(e));
    return OEQ_OK;
}

oeq_status oeq_sender_view(int64_t n_nodes, int64_t n_edges, const int32_t *rowptr, const int32_t *src, int32_t *srowptr,
                           int32_t *sperm, int32_t *sdst, void *workspace, size_t workspace_bytes, void *stream) {
    if (n_nodes < 0 || n_edges < 0) return fail(OEQ_ERR_INVALID_ARG, "negative size");
    if (n_nodes >= std::numeric_limits<int32_t>::max() || n_edges >= std::numeric_limits<int32_t>::max())
        return fail(OEQ_ERR_UNSUPPORTED, "sizes must fit int32");
    if (n_nodes == 0 && n_edges != 0) return fail(OEQ_ERR_INVALID_ARG, "edges without nodes");
    if (!srowptr || (n_edges > 0 && (!rowptr || !src || !sperm || !sdst))) return fail(OEQ_ERR_INVALID_ARG, "NULL array");
    size_t need = 0;
    oeq_status st = oeq_csr_workspace_size(n_nodes, n_edges, &need);
    if (st != OEQ_OK) return st;
    if (!workspace || workspace_bytes < need) return fail(OEQ_ERR_WORKSPACE, "workspace too small");
    if (reinterpret_cast<uintptr_t>(workspace) % kAlign)
        return fail(OEQ_ERR_WORKSPACE, "workspace must be 256-byte aligned");
    const hipError_t e = oeq::sender_view(n_nodes, n_edges, rowptr, src, srowptr, sperm, sdst, workspace,
                                          static_cast<hipStream_t>(stream));
    if (e != hipSuccess) return fail(OEQ_ERR_HIP, hipGetErrorString(e));
    return OEQ_OK;
}

oeq_status oeq_tp_conv_fwd_sender(const oeq_plan *plan, int64_t N, int64_t E, const int32_t *srowptr,
                                  const int32_t *sperm, const int32_t *sdst, const void *x, const void *Y,
                                  const void *W, void *out, void *stream) {
    oeq_status st = check_graph(plan, N, E, srowptr, sperm);
    if (st != OEQ_OK) return st;
    if ((st = check_channelwise(plan, "the sender forward")) != OEQ_OK) return st;
    if (E > 0 && !sdst) return fail(OEQ_ERR_INVALID_ARG, "sdst is NULL");
    if (N > 0 && !out) return fail(OEQ_ERR_INVALID_ARG, "out is NULL");
    if (E > 0 && (!x || !Y || !W)) return fail(OEQ_ERR_INVALID_ARG, "x, Y or W is NULL");
    oeq_plan *p = const_cast<oeq_plan *>(plan);
    hipStream_t s = static_cast<hipStream_t>(stream);
    if ((st = fill_zero(p, out, N * p->OD, s)) != OEQ_OK || E == 0) return st;
    int n_nodes = static_cast<int>(N);
    void *args[] = {&srowptr, &sperm, &sdst, &x, &Y, &W, &out, &n_nodes};
    if ((st = launch(p, "oeq_fwd_sender", static_cast<unsigned>(N), fwd_block(p), s, args)) != OEQ_OK) return st;
    void *uargs[] = {&out};
    return launch(p, "oeq_out_untranspose", static_cast<unsigned>(N), 256, s, uargs);
}

oeq_status oeq_tp_conv_bwd_sender(const oeq_plan *plan, int64_t N, int64_t E, const int32_t *srowptr,
                                  const int32_t *sperm, const int32_t *sdst, const void *x, const void *Y,
                                  const void *W, const void *g, void *gx, void *gY, void *gW, void *workspace,
                                  size_t workspace_bytes, void *stream) {
    oeq_status st = check_graph(plan, N, E, srowptr, sperm);
    if (st != OEQ_OK) return st;
    if ((st = check_channelwise(plan, "the sender VJP")) != OEQ_OK) return st;
    if (E > 0 && !sdst) return fail(OEQ_ERR_INVALID_ARG, "sdst is NULL");
    if (E > 0 && (!x || !Y || !W || !g)) return fail(OEQ_ERR_INVALID_ARG, "x, Y, W or grad_out is NULL");
    oeq_plan *p = const_cast<oeq_plan *>(plan);
    hipStream_t s = static_cast<hipStream_t>(stream);
    if (E == 0) return gx ? fill_zero(p, gx, N * p->XD, s) : OEQ_OK;
    if (!gx && !gY && !gW) return OEQ_OK;
    const bool gyp = gY && p->bwd_groups.size() > 1;
    Workspace w;
    if ((st = ws_bind(p, N, E, false, gyp, workspace, workspace_bytes, &w)) != OEQ_OK) return st;
    // an x block that feeds no path has a zero gradient that no group writes
    if (gx && p->x_unused && (st = fill_zero(p, gx, N * p->XD, s)) != OEQ_OK) return st;
    int flags = (gW ? 1 : 0) | (gY ? 2 : 0) | (gx ? 4 : 0);
    void *gy_target = gyp ? w.gy_part : gY;
    int64_t gy_stride = gyp ? E * p->YD : 0;
    const unsigned grid = static_cast<unsigned>(N * static_cast<int64_t>(p->bwd_groups.size()));
    int n_nodes = static_cast<int>(N);
    void *args[] = {&srowptr, &sperm, &sdst, &x, &Y, &W, &g, &gx, &gy_target, &gW, &flags, &gy_stride, &n_nodes};
    if ((st = launch(p, "oeq_bwd_sender", grid, bwd_block(p), s, args)) != OEQ_OK) return st;
    return gyp ? gy_combine(p, w, gY, E, s) : OEQ_OK;
}

oeq_status oeq_csr_check(int64_t n_nodes, int64_t n_edges, const int32_t *rowptr, const int32_t *src, void *stream) {
    if (n_nodes < 0 || n_edges < 0 || !rowptr || (n_edges > 0 && !src))
        return fail(OEQ_ERR_INVALID_ARG, "bad arguments");
    int bad = 0;
    const hipError_t e = oeq::csr_check(n_nodes, n_edges, rowptr, src, static_cast<hipStream_t>(stream), &bad);
    if (e != hipSuccess) return fail(OEQ_ERR_HIP, hipGetErrorString(e));
    if (bad) return fail(OEQ_ERR_INVALID_ARG, "invalid CSR (mask " + std::to_string(bad) + ")");
    return OEQ_OK;
}

}  // extern "C"
