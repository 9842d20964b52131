// C ABI entry points of the per-edge steps around the convolution: spherical
// harmonics of edge vectors and the passes that take vectors, the radial-weight
// network, and the forward / VJP that form the radial weights in the kernel.
#include "capi_internal.hpp"

using namespace oeq::capi;

namespace {

// Harmonics of an edge vector have parity (-1)^l: a Y block of the other parity (a
// pseudotensor) cannot come from one.
oeq_status check_y_from_vectors(const oeq_plan *p) {
    if (!p) return fail(OEQ_ERR_INVALID_ARG, "plan is NULL");
    if (!p->y_natural)
        return fail(OEQ_ERR_UNSUPPORTED, "Y blocks of parity other than (-1)^l cannot be harmonics of vectors");
    return OEQ_OK;
}

}  // namespace

extern "C" {

oeq_status oeq_sph_harm(const oeq_plan *plan, int64_t E, const void *vec, void *Y, void *stream) {
    if (oeq_status st = check_y_from_vectors(plan); st != OEQ_OK) return st;
    if (E < 0) return fail(OEQ_ERR_INVALID_ARG, "negative edge count");
    if (E == 0) return OEQ_OK;
    if (!vec || !Y) return fail(OEQ_ERR_INVALID_ARG, "vec or Y is NULL");
    oeq_plan *p = const_cast<oeq_plan *>(plan);
    void *args[] = {&vec, &Y, &E};
    return edge_launch(p, "oeq_sph_harm", E, args, static_cast<hipStream_t>(stream));
}

oeq_status oeq_sph_harm_bwd(const oeq_plan *plan, int64_t E, const void *vec, const void *gY, void *gvec,
                            void *stream) {
    if (oeq_status st = check_y_from_vectors(plan); st != OEQ_OK) return st;
    if (E < 0) return fail(OEQ_ERR_INVALID_ARG, "negative edge count");
    if (E == 0) return OEQ_OK;
    if (!vec || !gY || !gvec) return fail(OEQ_ERR_INVALID_ARG, "vec, grad_Y or grad_vec is NULL");
    oeq_plan *p = const_cast<oeq_plan *>(plan);
    void *args[] = {&vec, &gY, &gvec, &E};
    return edge_launch(p, "oeq_sph_harm_bwd", E, args, static_cast<hipStream_t>(stream));
}

oeq_status oeq_tp_conv_fwd_vec(const oeq_plan *plan, int64_t N, int64_t E, const int32_t *rowptr,
                               const int32_t *src, const void *x, const void *vec, const void *W, void *out,
                               void *stream) {
    oeq_status st = check_graph(plan, N, E, rowptr, src);
    if (st != OEQ_OK) return st;
    if ((st = check_y_from_vectors(plan)) != OEQ_OK) return st;
    if (N > 0 && !out) return fail(OEQ_ERR_INVALID_ARG, "out is NULL");
    if (E > 0 && (!x || !vec || !W)) return fail(OEQ_ERR_INVALID_ARG, "x, vec or W is NULL");
    oeq_plan *p = const_cast<oeq_plan *>(plan);
    int n_nodes = static_cast<int>(N);
    void *args[] = {&rowptr, &src, &x, &vec, &W, &out, &n_nodes};
    return launch(p, "oeq_fwd_vec", static_cast<unsigned>(N), fwd_block(p), static_cast<hipStream_t>(stream), args);
}

oeq_status oeq_workspace_size_vec(const oeq_plan *p, int64_t N, int64_t E, oeq_bwd_mode mode, size_t *bytes) {
    size_t base = 0;
    oeq_status st = oeq_workspace_size(p, N, E, mode, &base);
    if (st != OEQ_OK) return st;
    const size_t rows = up(static_cast<size_t>(E) * p->YD * esize(p));
    *bytes = 2 * rows + base;  // Y rows, Y-gradient rows, then the VJP's own workspace
    return OEQ_OK;
}

oeq_status oeq_tp_conv_bwd_vec(const oeq_plan *plan, int64_t N, int64_t E, const int32_t *rowptr,
                               const int32_t *src, const void *x, const void *vec, const void *W, const void *g,
                               void *gx, void *gvec, void *gW, oeq_bwd_mode mode, void *workspace,
                               size_t workspace_bytes, void *stream) {
    oeq_status st = check_graph(plan, N, E, rowptr, src);
    if (st != OEQ_OK) return st;
    if ((st = check_y_from_vectors(plan)) != OEQ_OK) return st;
    if (mode != OEQ_BWD_ATOMIC && mode != OEQ_BWD_DETERMINISTIC) return fail(OEQ_ERR_INVALID_ARG, "unknown mode");
    if (E > 0 && (!x || !vec || !W || !g)) return fail(OEQ_ERR_INVALID_ARG, "x, vec, W or grad_out is NULL");
    oeq_plan *p = const_cast<oeq_plan *>(plan);
    hipStream_t s = static_cast<hipStream_t>(stream);
    if (E == 0) return gx ? fill_zero(p, gx, N * p->XD, s) : OEQ_OK;
    if (!gx && !gvec && !gW) return OEQ_OK;
    size_t need = 0;
    if ((st = oeq_workspace_size_vec(p, N, E, mode, &need)) != OEQ_OK) return st;
    if (!workspace || workspace_bytes < need) return fail(OEQ_ERR_WORKSPACE, "workspace too small");
    if (reinterpret_cast<uintptr_t>(workspace) % kAlign)
        return fail(OEQ_ERR_WORKSPACE, "workspace must be 256-byte aligned");
    char *ws = static_cast<char *>(workspace);
    const size_t rows = up(static_cast<size_t>(E) * p->YD * esize(p));
    void *Yw = ws, *gYw = gvec ? ws + rows : nullptr;
    if ((st = oeq_sph_harm(p, E, vec, Yw, stream)) != OEQ_OK) return st;
    if ((st = oeq_tp_conv_bwd(p, N, E, rowptr, src, x, Yw, W, g, gx, gYw, gW, mode, ws + 2 * rows,
                              workspace_bytes - 2 * rows, stream)) != OEQ_OK)
        return st;
    return gvec ? oeq_sph_harm_bwd(p, E, vec, gYw, gvec, stream) : OEQ_OK;
}

oeq_status oeq_tp_conv_fwd_pos(const oeq_plan *plan, int64_t N, int64_t E, const int32_t *rowptr,
                               const int32_t *src, const void *x, const void *pos, const void *W, void *out,
                               void *stream) {
    oeq_status st = check_graph(plan, N, E, rowptr, src);
    if (st != OEQ_OK) return st;
    if ((st = check_y_from_vectors(plan)) != OEQ_OK) return st;
    if (N > 0 && !out) return fail(OEQ_ERR_INVALID_ARG, "out is NULL");
    if (E > 0 && (!x || !pos || !W)) return fail(OEQ_ERR_INVALID_ARG, "x, pos or W is NULL");
    oeq_plan *p = const_cast<oeq_plan *>(plan);
    int n_nodes = static_cast<int>(N);
    void *args[] = {&rowptr, &src, &x, &pos, &W, &out, &n_nodes};
    return launch(p, "oeq_fwd_pos", static_cast<unsigned>(N), fwd_block(p), static_cast<hipStream_t>(stream), args);
}

namespace {

// Workspace of the VJP from positions: edge vectors [E, 3], Y rows, Y-gradient rows,
// vector gradients [E, 3], the sender CSR (deterministic mode), then the VJP's own.
struct PosWs {
    size_t vec = 0, Y = 0, gY = 0, gvec = 0, srowptr = 0, sperm = 0, csr = 0, vjp = 0, bytes = 0;
};

oeq_status pos_layout(const oeq_plan *p, int64_t N, int64_t E, oeq_bwd_mode mode, PosWs *w) {
    const size_t es = esize(p), e = static_cast<size_t>(E);
    size_t off = 0;
    w->vec = off;
    off += up(e * 3 * es);
    w->Y = off;
    off += up(e * p->YD * es);
    w->gY = off;
    off += up(e * p->YD * es);
    w->gvec = off;
    off += up(e * 3 * es);
    if (mode == OEQ_BWD_DETERMINISTIC) {
        size_t csr = 0;
        const hipError_t he = oeq::sender_csr_workspace(N, E, &csr);
        if (he != hipSuccess) return fail(OEQ_ERR_HIP, std::string("sender CSR workspace: ") + hipGetErrorString(he));
        w->srowptr = off;
        off += up(sizeof(int32_t) * static_cast<size_t>(N + 1));
        w->sperm = off;
        off += up(sizeof(int32_t) * (e > 0 ? e : 1));
        w->csr = off;
        off += up(csr);
    }
    size_t base = 0;
    oeq_status st = oeq_workspace_size(p, N, E, mode, &base);
    if (st != OEQ_OK) return st;
    w->vjp = off;
    w->bytes = off + base;
    return OEQ_OK;
}

}  // namespace

oeq_status oeq_workspace_size_pos(const oeq_plan *p, int64_t N, int64_t E, oeq_bwd_mode mode, size_t *bytes) {
    if (!p || !bytes) return fail(OEQ_ERR_INVALID_ARG, "plan or output is NULL");
    if (N < 0 || E < 0) return fail(OEQ_ERR_INVALID_ARG, "negative size");
    if (mode != OEQ_BWD_ATOMIC && mode != OEQ_BWD_DETERMINISTIC) return fail(OEQ_ERR_INVALID_ARG, "unknown mode");
    PosWs w;
    oeq_status st = pos_layout(p, N, E, mode, &w);
    if (st != OEQ_OK) return st;
    *bytes = w.bytes;
    return OEQ_OK;
}

oeq_status oeq_tp_conv_bwd_pos(const oeq_plan *plan, int64_t N, int64_t E, const int32_t *rowptr,
                               const int32_t *src, const void *x, const void *pos, const void *W, const void *g,
                               void *gx, void *gpos, void *gW, oeq_bwd_mode mode, void *workspace,
                               size_t workspace_bytes, void *stream) {
    oeq_status st = check_graph(plan, N, E, rowptr, src);
    if (st != OEQ_OK) return st;
    if ((st = check_y_from_vectors(plan)) != OEQ_OK) return st;
    if (mode != OEQ_BWD_ATOMIC && mode != OEQ_BWD_DETERMINISTIC) return fail(OEQ_ERR_INVALID_ARG, "unknown mode");
    if (E > 0 && (!x || !pos || !W || !g)) return fail(OEQ_ERR_INVALID_ARG, "x, pos, W or grad_out is NULL");
    oeq_plan *p = const_cast<oeq_plan *>(plan);
    hipStream_t s = static_cast<hipStream_t>(stream);
    if (E == 0) {
        if (gx && (st = fill_zero(p, gx, N * p->XD, s)) != OEQ_OK) return st;
        return gpos ? fill_zero(p, gpos, N * 3, s) : OEQ_OK;
    }
    if (!gx && !gpos && !gW) return OEQ_OK;
    PosWs w;
    if ((st = pos_layout(p, N, E, mode, &w)) != OEQ_OK) return st;
    if (!workspace || workspace_bytes < w.bytes) return fail(OEQ_ERR_WORKSPACE, "workspace smaller than oeq_workspace_size_pos");
    if (reinterpret_cast<uintptr_t>(workspace) % kAlign)
        return fail(OEQ_ERR_WORKSPACE, "workspace must be 256-byte aligned");
    char *ws = static_cast<char *>(workspace);
    void *vec = ws + w.vec, *Yw = ws + w.Y, *gYw = gpos ? ws + w.gY : nullptr, *gvec = ws + w.gvec;
    int n_nodes = static_cast<int>(N);
    void *yargs[] = {&rowptr, &src, &pos, &Yw, &vec, &n_nodes};
    if ((st = launch(p, "oeq_sph_harm_pos", static_cast<unsigned>(N), 64, s, yargs)) != OEQ_OK) return st;
    if ((st = oeq_tp_conv_bwd(p, N, E, rowptr, src, x, Yw, W, g, gx, gYw, gW, mode, ws + w.vjp,
                              workspace_bytes - w.vjp, stream)) != OEQ_OK)
        return st;
    if (!gpos) return OEQ_OK;
    void *gargs[] = {&vec, &gYw, &gvec, &E};
    if ((st = edge_launch(p, "oeq_sph_harm_bwd", E, gargs, s)) != OEQ_OK) return st;
    if (mode == OEQ_BWD_ATOMIC) {
        if ((st = fill_zero(p, gpos, N * 3, s)) != OEQ_OK) return st;
        void *args[] = {&rowptr, &src, &gvec, &gpos, &n_nodes};
        return launch(p, "oeq_pos_scatter_atomic", static_cast<unsigned>(N), 64, s, args);
    }
    int32_t *srp = reinterpret_cast<int32_t *>(ws + w.srowptr), *spm = reinterpret_cast<int32_t *>(ws + w.sperm);
    const hipError_t he = oeq::sender_csr(N, E, src, srp, spm, ws + w.csr, s);
    if (he != hipSuccess) return fail(OEQ_ERR_HIP, std::string("sender CSR: ") + hipGetErrorString(he));
    void *args[] = {&rowptr, &srp, &spm, &gvec, &gpos, &n_nodes};
    const unsigned blocks = static_cast<unsigned>(std::min<int64_t>((N + 255) / 256, 65536));
    return launch(p, "oeq_pos_scatter_det", blocks, 256, s, args);
}

oeq_status oeq_radial_workspace_size(const oeq_plan *p, int64_t E, int32_t hidden, size_t *bytes) {
    if (!p || !bytes) return fail(OEQ_ERR_INVALID_ARG, "plan or output is NULL");
    if (E < 0 || hidden < 1 || hidden > 1024) return fail(OEQ_ERR_INVALID_ARG, "bad size");
    *bytes = radial_layout(p, E, hidden).bytes;
    return OEQ_OK;
}

oeq_status oeq_radial_fwd(const oeq_plan *plan, int64_t E, const void *vec, double r_cut, int32_t hidden,
                          const void *W1, const void *W2, void *W, void *workspace, size_t workspace_bytes,
                          void *stream) {
    RadialWs w;
    oeq_status st = radial_check(plan, E, r_cut, hidden, vec, W1, W2, workspace, workspace_bytes, &w);
    if (st != OEQ_OK) return st;
    if (E == 0) return OEQ_OK;
    if (!W) return fail(OEQ_ERR_INVALID_ARG, "W is NULL");
    oeq_plan *p = const_cast<oeq_plan *>(plan);
    hipStream_t s = static_cast<hipStream_t>(stream);
    char *ws = static_cast<char *>(workspace);
    if ((st = radial_hidden(p, E, vec, r_cut, hidden, W1, ws, w, s)) != OEQ_OK) return st;
    const int PU = static_cast<int>(p->paths.size()) * p->U;
    return gemm(p, static_cast<int>(E), PU, hidden, ws + w.h, hidden, false, W2, PU, false, W, PU,
                1.0 / std::sqrt(static_cast<double>(hidden)), 1, nullptr, s);
}

oeq_status oeq_radial_bwd(const oeq_plan *plan, int64_t E, const void *vec, double r_cut, int32_t hidden,
                          const void *W1, const void *W2, const void *gW, void *gvec, void *gW1, void *gW2,
                          void *workspace, size_t workspace_bytes, void *stream) {
    RadialWs w;
    oeq_status st = radial_check(plan, E, r_cut, hidden, vec, W1, W2, workspace, workspace_bytes, &w);
    if (st != OEQ_OK) return st;
    oeq_plan *p = const_cast<oeq_plan *>(plan);
    hipStream_t s = static_cast<hipStream_t>(stream);
    const int H = hidden, PU = static_cast<int>(p->paths.size()) * p->U;
    if (E == 0) {  // sums over no edges
        if (gW1 && (st = fill_zero(p, gW1, int64_t(kRadialNB) * H, s)) != OEQ_OK) return st;
        return gW2 ? fill_zero(p, gW2, int64_t(H) * PU, s) : OEQ_OK;
    }
    if (!gW) return fail(OEQ_ERR_INVALID_ARG, "grad_W is NULL");
    if (!gvec && !gW1 && !gW2) return OEQ_OK;
    char *ws = static_cast<char *>(workspace);
    const int Ei = static_cast<int>(E);
    const double sh = 1.0 / std::sqrt(static_cast<double>(H)), s8 = 1.0 / std::sqrt(double(kRadialNB));
    if ((st = radial_hidden(p, E, vec, r_cut, H, W1, ws, w, s)) != OEQ_OK) return st;
    // gW2 = h^T gW / sqrt(H): a sum over edges
    if (gW2 && (st = gemm(p, H, PU, Ei, ws + w.h, H, true, gW, PU, false, gW2, PU, sh, w.splitsW2, ws + w.pW2, s)) !=
                   OEQ_OK)
        return st;
    if (!gvec && !gW1) return OEQ_OK;
    // dh = gW W2^T / sqrt(H), then dpre = dh silu'(pre) in place
    void *dh = ws + w.dh, *Bp = ws + w.B;
    if ((st = gemm(p, Ei, H, PU, gW, PU, false, W2, PU, true, dh, H, sh, 1, nullptr, s)) != OEQ_OK) return st;
    void *dargs[] = {&Bp, &W1, const_cast<int *>(&H), &dh, &E};
    if ((st = edge_launch(p, "oeq_radial_dpre", E * H, dargs, s)) != OEQ_OK) return st;
    // gW1 = B^T dpre / sqrt(8): a sum over edges
    if (gW1 && (st = gemm(p, kRadialNB, H, Ei, Bp, kRadialNB, true, dh, H, false, gW1, H, s8, w.splitsW1,
                          ws + w.pW1, s)) != OEQ_OK)
        return st;
    if (!gvec) return OEQ_OK;
    // dB = dpre W1^T / sqrt(8), then the chain through r = |vec|
    void *dB = ws + w.dB;
    if ((st = gemm(p, Ei, kRadialNB, H, dh, H, false, W1, H, true, dB, kRadialNB, s8, 1, nullptr, s)) != OEQ_OK)
        return st;
    float rcf = static_cast<float>(r_cut);
    void *rc = p->dtype == OEQ_F64 ? static_cast<void *>(&r_cut) : static_cast<void *>(&rcf);
    void *gargs[] = {&vec, rc, &dB, &gvec, &E};
    return edge_launch(p, "oeq_radial_gvec", E, gargs, s);
}

oeq_status oeq_tp_conv_fwd_radial(const oeq_plan *plan, int64_t N, int64_t E, const int32_t *rowptr,
                                  const int32_t *src, const void *x, const void *Y, const void *vec, double r_cut,
                                  const void *W1, const void *W2, void *out, void *workspace, size_t workspace_bytes,
                                  void *stream) {
    oeq_status st = check_graph(plan, N, E, rowptr, src);
    if (st != OEQ_OK) return st;
    if ((st = check_channelwise(plan, "the forward with in-kernel radial weights")) != OEQ_OK) return st;
    if (N > 0 && !out) return fail(OEQ_ERR_INVALID_ARG, "out is NULL");
    if (E > 0 && (!x || !Y)) return fail(OEQ_ERR_INVALID_ARG, "x or Y is NULL");
    RadialWs w;
    if ((st = radial_check(plan, E, r_cut, kFusedHidden, vec, W1, W2, workspace, workspace_bytes, &w)) != OEQ_OK)
        return st;
    oeq_plan *p = const_cast<oeq_plan *>(plan);
    hipStream_t s = static_cast<hipStream_t>(stream);
    if (E == 0) return fill_zero(p, out, N * p->OD, s);  // no edges: W2 and the workspace are not read
    char *ws = static_cast<char *>(workspace);
    if ((st = radial_hidden(p, E, vec, r_cut, kFusedHidden, W1, ws, w, s)) != OEQ_OK) return st;
    void *hid = ws + w.h;
    int n_nodes = static_cast<int>(N);
    void *args[] = {&rowptr, &src, &x, &Y, &hid, &W2, &out, &n_nodes};
    return launch(p, "oeq_fwd_radial", static_cast<unsigned>(N), fwd_block(p), s, args);
}

}  // extern "C"

namespace {
// the rest of the radial backward from dh (E x 8 in the workspace): dpre = dh silu'(pre) in
// place, gW1 = B^T dpre / sqrt(8), dB = dpre W1^T / sqrt(8), then grad_vec through r = |vec|
oeq_status radial_vjp_tail(oeq_plan *p, int64_t E, const void *vec, double r_cut, const void *W1, void *gvec,
                           void *gW1, char *ws, const RadialWs &w, hipStream_t s) {
    if (!gvec && !gW1) return OEQ_OK;
    oeq_status st;
    const int H = kFusedHidden, Ei = static_cast<int>(E);
    const double s8 = 1.0 / std::sqrt(double(kRadialNB));
    void *Bp = ws + w.B, *dh = ws + w.dh;
    void *dargs[] = {&Bp, &W1, const_cast<int *>(&H), &dh, &E};
    if ((st = edge_launch(p, "oeq_radial_dpre", E * H, dargs, s)) != OEQ_OK) return st;
    if (gW1 && (st = gemm(p, kRadialNB, H, Ei, Bp, kRadialNB, true, dh, H, false, gW1, H, s8, w.splitsW1,
                          ws + w.pW1, s)) != OEQ_OK)
        return st;
    if (!gvec) return OEQ_OK;
    void *dB = ws + w.dB;
    if ((st = gemm(p, Ei, kRadialNB, H, dh, H, false, W1, H, true, dB, kRadialNB, s8, 1, nullptr, s)) != OEQ_OK)
        return st;
    float rcf = static_cast<float>(r_cut);
    void *rc = p->dtype == OEQ_F64 ? static_cast<void *>(&r_cut) : static_cast<void *>(&rcf);
    void *gargs[] = {&vec, rc, &dB, &gvec, &E};
    return edge_launch(p, "oeq_radial_gvec", E, gargs, s);
}
}  // namespace

extern "C" {

oeq_status oeq_workspace_size_radial(const oeq_plan *p, int64_t N, int64_t E, oeq_bwd_mode mode, size_t *bytes) {
    if (!p || !bytes) return fail(OEQ_ERR_INVALID_ARG, "plan or output is NULL");
    if (N < 0 || E < 0) return fail(OEQ_ERR_INVALID_ARG, "negative size");
    if (mode != OEQ_BWD_ATOMIC && mode != OEQ_BWD_DETERMINISTIC) return fail(OEQ_ERR_INVALID_ARG, "unknown mode");
    RadVjpWs w;
    oeq_status st = radvjp_layout(p, N, E, mode == OEQ_BWD_DETERMINISTIC, nullptr, &w);
    if (st != OEQ_OK) return st;
    *bytes = w.bytes;
    return OEQ_OK;
}

oeq_status oeq_tp_conv_bwd_radial(const oeq_plan *plan, int64_t N, int64_t E, const int32_t *rowptr,
                                  const int32_t *src, const void *x, const void *Y, const void *vec, double r_cut,
                                  const void *W1, const void *W2, const void *g, void *gx, void *gY, void *gvec,
                                  void *gW1, void *gW2, oeq_bwd_mode mode, void *workspace, size_t workspace_bytes,
                                  void *stream) {
    oeq_status st = check_graph(plan, N, E, rowptr, src);
    if (st != OEQ_OK) return st;
    if ((st = check_channelwise(plan, "the VJP with in-kernel radial weights")) != OEQ_OK) return st;
    if (mode != OEQ_BWD_ATOMIC && mode != OEQ_BWD_DETERMINISTIC) return fail(OEQ_ERR_INVALID_ARG, "unknown mode");
    if (E > 0 && (!x || !Y || !g)) return fail(OEQ_ERR_INVALID_ARG, "x, Y or grad_out is NULL");
    oeq_plan *p = const_cast<oeq_plan *>(plan);
    if (p->YD < kFusedHidden) return fail(OEQ_ERR_UNSUPPORTED, "the radial VJP needs Y degrees up to at least 2");
    RadialWs rw;
    if ((st = radial_check(plan, E, r_cut, kFusedHidden, vec, W1, W2, nullptr, 0, &rw)) != OEQ_OK &&
        st != OEQ_ERR_WORKSPACE)
        return st;
    hipStream_t s = static_cast<hipStream_t>(stream);
    const int H = kFusedHidden, PU = static_cast<int>(p->paths.size()) * p->U;
    if (E == 0) {
        if (gx && (st = fill_zero(p, gx, N * p->XD, s)) != OEQ_OK) return st;
        if (gW1 && (st = fill_zero(p, gW1, int64_t(kRadialNB) * H, s)) != OEQ_OK) return st;
        return gW2 ? fill_zero(p, gW2, int64_t(H) * PU, s) : OEQ_OK;
    }
    if (!gx && !gY && !gvec && !gW1 && !gW2) return OEQ_OK;
    const bool det = gx && mode == OEQ_BWD_DETERMINISTIC;
    RadVjpWs w;
    if ((st = radvjp_layout(p, N, E, det, static_cast<char *>(workspace), &w)) != OEQ_OK) return st;
    if (!workspace || workspace_bytes < w.bytes) return fail(OEQ_ERR_WORKSPACE, "workspace too small");
    if (reinterpret_cast<uintptr_t>(workspace) % kAlign)
        return fail(OEQ_ERR_WORKSPACE, "workspace must be 256-byte aligned");
    char *ws = static_cast<char *>(workspace);
    if ((st = radial_hidden(p, E, vec, r_cut, H, W1, ws, w.rad, s)) != OEQ_OK) return st;
    const int G = static_cast<int>(p->rad_groups.size());
    const bool want_dh = gvec || gW1;
    const int Ei = static_cast<int>(E);
    const double s8 = 1.0 / std::sqrt(double(kRadialNB));
    void *hid = ws + w.rad.h, *dh = ws + w.rad.dh;
    if (p->rad_compose) {
        // W = h W2 / sqrt(8) per edge, the convolution VJP, then gW2 = h^T gW / sqrt(8) and
        // dh = gW W2^T / sqrt(8): the same sums with W and its gradient held in the workspace
        void *Wb = ws + w.wbuf, *gWb = (gW2 || want_dh) ? ws + w.gwbuf : nullptr;
        if ((st = gemm(p, Ei, PU, H, hid, H, false, W2, PU, false, Wb, PU, s8, 1, nullptr, s)) != OEQ_OK) return st;
        if ((st = oeq_tp_conv_bwd(plan, N, E, rowptr, src, x, Y, Wb, g, gx, gY, gWb, mode, ws + w.conv_off,
                                  w.conv.bytes, stream)) != OEQ_OK)
            return st;
        if (gW2 && (st = gemm(p, H, PU, Ei, hid, H, true, gWb, PU, false, gW2, PU, s8, w.rad.splitsW2,
                              ws + w.rad.pW2, s)) != OEQ_OK)
            return st;
        if (want_dh && (st = gemm(p, Ei, H, PU, gWb, PU, false, W2, PU, true, dh, H, s8, 1, nullptr, s)) != OEQ_OK)
            return st;
        return radial_vjp_tail(p, E, vec, r_cut, W1, gvec, gW1, ws, w.rad, s);
    }
    int flags = (gW2 ? 1 : 0) | (gY ? 2 : 0) | (want_dh ? 4 : 0);
    void *w2p = ws + w.w2p;
    void *gy_target = G > 1 ? ws + w.gyp : gY, *dh_target = G > 1 ? ws + w.dhp : dh;
    int64_t gy_stride = G > 1 ? E * p->YD : 0, dh_stride = G > 1 ? E * H : 0;
    const unsigned grid = static_cast<unsigned>(N * static_cast<int64_t>(G));
    const unsigned block = bwd_block(p);
    int n_nodes = static_cast<int>(N);
    if (!gx) {
        void *args[] = {&rowptr, &src, &x, &Y, &hid, &W2, &g, &gx, &gy_target, &dh_target, &w2p, &flags, &gy_stride,
                        &dh_stride, &n_nodes};
        if ((st = launch(p, "oeq_bwd_radial_nogx", grid, block, s, args)) != OEQ_OK) return st;
    } else if (!det) {
        if ((st = fill_zero(p, gx, N * p->XD, s)) != OEQ_OK) return st;
        void *args[] = {&rowptr, &src, &x, &Y, &hid, &W2, &g, &gx, &gy_target, &dh_target, &w2p, &flags, &gy_stride,
                        &dh_stride, &n_nodes};
        if ((st = launch(p, "oeq_bwd_radial_atomic", grid, block, s, args)) != OEQ_OK) return st;
        if ((st = untranspose(p, N, gx, s)) != OEQ_OK) return st;
    } else {
        if ((st = sender_csr_into(N, E, src, w.conv, s)) != OEQ_OK) return st;
        void *hrows = w.conv.h;
        // each group writes the x blocks of its own paths; a block no path uses stays zero
        if (p->x_unused && (st = fill_zero(p, hrows, E * p->XD, s)) != OEQ_OK) return st;
        void *args[] = {&rowptr, &src, &x, &Y, &hid, &W2, &g, &hrows, &gy_target, &dh_target, &w2p, &flags,
                        &gy_stride, &dh_stride, &n_nodes};
        if ((st = launch(p, "oeq_bwd_radial_rows", grid, block, s, args)) != OEQ_OK) return st;
        if ((st = det_finish(p, N, w.conv, gx, s)) != OEQ_OK) return st;
    }
    if (G > 1) {
        if (gY && (st = combine_parts(p, gy_target, G, gY, E * p->YD, s)) != OEQ_OK) return st;
        if (want_dh && (st = combine_parts(p, dh_target, G, dh, E * H, s)) != OEQ_OK) return st;
    }
    // sum of the receivers' partial rows, in receiver order
    if (gW2 && (st = ordered_sum(p, w2p, static_cast<int>(N), kFusedHidden, PU, gW2, PU, ws + w.w2s, s)) != OEQ_OK)
        return st;
    return radial_vjp_tail(p, E, vec, r_cut, W1, gvec, gW1, ws, w.rad, s);
}

}  // extern "C"
