// C ABI entry points of the plans and the receiver-stationary convolution passes
// (forward, VJP, double backward): argument checks on the host only (no device
// reads, no synchronisation), workspace carving and stream-ordered launches.
#include <cstdio>

#include "capi_internal.hpp"
#include "noalloc.hpp"

using namespace oeq::capi;

extern "C" {


const char *oeq_status_string(oeq_status s) {
    switch (s) {
    case OEQ_OK: return "OEQ_OK";
    case OEQ_ERR_INVALID_ARG: return "OEQ_ERR_INVALID_ARG";
    case OEQ_ERR_UNSUPPORTED: return "OEQ_ERR_UNSUPPORTED";
    case OEQ_ERR_WORKSPACE: return "OEQ_ERR_WORKSPACE";
    case OEQ_ERR_HIP: return "OEQ_ERR_HIP";
    case OEQ_ERR_JIT: return "OEQ_ERR_JIT";
    }
    return "unknown oeq_status";
}

const char *oeq_last_error(void) { return g_last_error.c_str(); }

namespace {

oeq_status plan_create(const oeq_tp_desc *desc, oeq_plan **plan, bool cache_only) {
    if (!plan) return fail(OEQ_ERR_INVALID_ARG, "plan output pointer is NULL");
    *plan = nullptr;
    oeq_plan *p = new oeq_plan();
    std::string why;
    oeq_status st = oeq::plan_build(desc, p, &why);
    if (st == OEQ_OK) {
        p->source = oeq::emit_source(*p);
        st = oeq::jit_compile(*p, &why, cache_only);
    }
    if (st != OEQ_OK) {
        delete p;
        return fail(st, why);
    }
    *plan = p;
    return OEQ_OK;
}

}  // namespace

oeq_status oeq_plan_create(const oeq_tp_desc *desc, oeq_plan **plan) { return plan_create(desc, plan, false); }

oeq_status oeq_plan_create_cached(const oeq_tp_desc *desc, oeq_plan **plan) { return plan_create(desc, plan, true); }

void oeq_plan_destroy(oeq_plan *plan) {
    if (!plan) return;
    for (auto &kv : plan->modules)
        if (kv.second.module) {
            int cur = 0;
            if (hipGetDevice(&cur) == hipSuccess && hipSetDevice(kv.first) == hipSuccess) {
                (void)hipModuleUnload(kv.second.module);
                (void)hipSetDevice(cur);
            }
        }
    delete plan;
}

oeq_status oeq_plan_dims(const oeq_plan *p, int64_t *x_dim, int64_t *y_dim, int64_t *out_dim, int64_t *n_paths,
                         int64_t *w_per_edge) {
    if (!p) return fail(OEQ_ERR_INVALID_ARG, "plan is NULL");
    if (x_dim) *x_dim = p->XD;
    if (y_dim) *y_dim = p->YD;
    if (out_dim) *out_dim = p->OD;
    if (n_paths) *n_paths = static_cast<int64_t>(p->paths.size());
    if (w_per_edge) *w_per_edge = static_cast<int64_t>(p->paths.size()) * p->U;
    return OEQ_OK;
}

oeq_status oeq_plan_paths(const oeq_plan *p, int32_t *out6, int32_t capacity) {
    if (!p || !out6) return fail(OEQ_ERR_INVALID_ARG, "plan or output is NULL");
    if (capacity < static_cast<int32_t>(p->paths.size())) return fail(OEQ_ERR_INVALID_ARG, "capacity too small");
    for (size_t k = 0; k < p->paths.size(); ++k) {
        const auto &pa = p->paths[k];
        int32_t *o = out6 + 6 * k;
        o[0] = pa.i1;
        o[1] = pa.l1;
        o[2] = pa.l2;
        o[3] = pa.l3;
        o[4] = pa.ob;
        o[5] = pa.parity3;
    }
    return OEQ_OK;
}

oeq_status oeq_plan_code_key(const oeq_plan *p, char *buf, size_t len) {
    if (!p || !buf) return fail(OEQ_ERR_INVALID_ARG, "plan or buffer is NULL");
    if (len < p->code_key.size() + 1) return fail(OEQ_ERR_INVALID_ARG, "buffer too small");
    std::memcpy(buf, p->code_key.c_str(), p->code_key.size() + 1);
    return OEQ_OK;
}

oeq_status oeq_cg_table(int32_t l1, int32_t l2, int32_t l3, double *out) {
    if (!out) return fail(OEQ_ERR_INVALID_ARG, "output is NULL");
    std::vector<double> t;
    if (!oeq::cg_real_table(l1, l2, l3, t)) return fail(OEQ_ERR_INVALID_ARG, "no table for these degrees");
    std::memcpy(out, t.data(), sizeof(double) * t.size());
    return OEQ_OK;
}

oeq_status oeq_workspace_size(const oeq_plan *p, int64_t n_nodes, int64_t n_edges, oeq_bwd_mode mode,
                              size_t *bytes) {
    if (!p || !bytes) return fail(OEQ_ERR_INVALID_ARG, "plan or output is NULL");
    if (n_nodes < 0 || n_edges < 0) return fail(OEQ_ERR_INVALID_ARG, "negative size");
    if (mode != OEQ_BWD_ATOMIC && mode != OEQ_BWD_DETERMINISTIC) return fail(OEQ_ERR_INVALID_ARG, "unknown mode");
    // the VJP's sender-stationary route (when the plan takes it) needs the sender view
    return vjp_ws_bytes(p, n_nodes, n_edges, mode, bytes);
}

oeq_status oeq_tp_conv_fwd(const oeq_plan *plan, int64_t N, int64_t E, const int32_t *rowptr, const int32_t *src,
                           const void *x, const void *Y, const void *W, void *out, void *stream) {
    oeq_status st = check_graph(plan, N, E, rowptr, src);
    if (st != OEQ_OK) return st;
    if (N > 0 && !out) return fail(OEQ_ERR_INVALID_ARG, "out is NULL");
    if (E > 0 && (!x || !Y || !W)) return fail(OEQ_ERR_INVALID_ARG, "x, Y or W is NULL");
    return fwd_launch(const_cast<oeq_plan *>(plan), N, rowptr, src, x, Y, W, out, 0, static_cast<hipStream_t>(stream));
}

oeq_status oeq_tp_conv_bwd(const oeq_plan *plan, int64_t N, int64_t E, const int32_t *rowptr, const int32_t *src,
                           const void *x, const void *Y, const void *W, const void *g, void *gx, void *gY, void *gW,
                           oeq_bwd_mode mode, void *workspace, size_t workspace_bytes, void *stream) {
    oeq_status st = check_graph(plan, N, E, rowptr, src);
    if (st != OEQ_OK) return st;
    if (mode != OEQ_BWD_ATOMIC && mode != OEQ_BWD_DETERMINISTIC) return fail(OEQ_ERR_INVALID_ARG, "unknown mode");
    if (E > 0 && (!x || !Y || !W || !g)) return fail(OEQ_ERR_INVALID_ARG, "x, Y, W or grad_out is NULL");
    oeq_plan *p = const_cast<oeq_plan *>(plan);
    hipStream_t s = static_cast<hipStream_t>(stream);
    if (E == 0) return gx ? fill_zero(p, gx, N * p->XD, s) : OEQ_OK;
    if (!gx && !gY && !gW) return OEQ_OK;
    if (bwd_by_sender(p, E)) {
        // the plan's data-movement model prefers the sender-stationary pass ("source
        // stationary"): the sender view goes into the workspace, then the pass runs
        SenderWs sw;
        if ((st = sender_ws_layout(p, N, E, &sw)) != OEQ_OK) return st;
        if (!workspace || workspace_bytes < sw.bytes)
            return fail(OEQ_ERR_WORKSPACE, "workspace smaller than oeq_workspace_size");
        if (reinterpret_cast<uintptr_t>(workspace) % kAlign)
            return fail(OEQ_ERR_WORKSPACE, "workspace must be 256-byte aligned");
        char *ws = static_cast<char *>(workspace);
        int32_t *srp = reinterpret_cast<int32_t *>(ws + sw.srowptr), *spm = reinterpret_cast<int32_t *>(ws + sw.sperm),
                *sdst = reinterpret_cast<int32_t *>(ws + sw.sdst);
        const hipError_t he = oeq::sender_view(N, E, rowptr, src, srp, spm, sdst, ws + sw.csr, s);
        if (he != hipSuccess) return fail(OEQ_ERR_HIP, std::string("sender view: ") + hipGetErrorString(he));
        return oeq_tp_conv_bwd_sender(plan, N, E, srp, spm, sdst, x, Y, W, g, gx, gY, gW, ws + sw.vjp,
                                      workspace_bytes - sw.vjp, stream);
    }
    const bool det = gx && mode == OEQ_BWD_DETERMINISTIC;
    const bool gyp = gY && p->bwd_groups.size() > 1;
    const bool gxe = gx && needs_gxe(p);
    Workspace w;
    if ((st = ws_bind(p, N, E, det, gyp, workspace, workspace_bytes, &w, gxe)) != OEQ_OK) return st;
    int flags = (gW ? 1 : 0) | (gY ? 2 : 0);
    void *gy_target = gyp ? w.gy_part : gY;
    int64_t gy_stride = gyp ? E * p->YD : 0;
    const unsigned grid = static_cast<unsigned>(N * static_cast<int64_t>(p->bwd_groups.size()));
    const unsigned block = bwd_block(p);
    int n_nodes = static_cast<int>(N);
    if (!gx) {
        void *args[] = {&rowptr, &src, &x, &Y, &W, &g, &gx, &gy_target, &gW, &flags, &gy_stride, &n_nodes};
        st = launch(p, "oeq_bwd_nogx", grid, block, s, args);
    } else if (mode == OEQ_BWD_ATOMIC) {
        void *gxr = gxe ? w.gxe : gx;  // rows of GXD values
        if ((st = fill_zero(p, gxr, N * p->GXD, s)) != OEQ_OK) return st;
        void *args[] = {&rowptr, &src, &x, &Y, &W, &g, &gxr, &gy_target, &gW, &flags, &gy_stride, &n_nodes};
        if ((st = launch(p, "oeq_bwd_atomic", grid, block, s, args)) != OEQ_OK) return st;
        if ((st = untranspose(p, N, gxr, s)) != OEQ_OK) return st;
        if (gxe) st = fold_x(p, N, gxr, gx, s);
    } else {
        if ((st = sender_csr_into(N, E, src, w, s)) != OEQ_OK) return st;
        void *h = w.h;
        // an x block that feeds no path is never written into the per-edge rows
        if (p->x_unused && (st = fill_zero(p, h, E * p->GXD, s)) != OEQ_OK) return st;
        void *args[] = {&rowptr, &src, &x, &Y, &W, &g, &h, &gy_target, &gW, &flags, &gy_stride, &n_nodes};
        if ((st = launch(p, "oeq_bwd_rows", grid, block, s, args)) != OEQ_OK) return st;
        st = det_finish(p, N, w, gx, s);
    }
    if (st != OEQ_OK) return st;
    return gyp ? gy_combine(p, w, gY, E, s) : OEQ_OK;
}

oeq_status oeq_tp_conv_bwd_noalloc(const oeq_plan *plan, int64_t N, int64_t E, const int32_t *rowptr,
                                   const int32_t *src, const void *x, const void *Y, const void *W, const void *g,
                                   void *gx, void *gY, void *gW, oeq_bwd_mode mode, void *stream) {
    oeq_status st = check_graph(plan, N, E, rowptr, src);
    if (st != OEQ_OK) return st;
    if (mode != OEQ_BWD_ATOMIC && mode != OEQ_BWD_DETERMINISTIC) return fail(OEQ_ERR_INVALID_ARG, "unknown mode");
    oeq_plan *p = const_cast<oeq_plan *>(plan);
    // the scratch this call binds: exactly what oeq_tp_conv_bwd carves from its workspace
    size_t need = 0;
    if ((st = bwd_ws_bytes(p, N, E, mode, gx != nullptr, gY != nullptr, &need)) != OEQ_OK) return st;
    if (need > oeq::kNoAllocScratchBytes) {
        char msg[160];
        std::snprintf(msg, sizeof msg, "this call needs %zu bytes of scratch; the allocation-free entry point holds %zu",
                      need, oeq::kNoAllocScratchBytes);
        return fail(OEQ_ERR_WORKSPACE, msg);
    }
    int dev = 0;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return fail(OEQ_ERR_HIP, std::string("hipGetDevice: ") + hipGetErrorString(e));
    // loading the plan's kernels on a device allocates device memory: an ordinary call
    // with this plan on this device must come first
    if (!oeq::module_loaded(*p, dev))
        return fail(OEQ_ERR_INVALID_ARG, "the plan's kernels are not loaded on this device yet (make one ordinary "
                                         "call with the plan on this device first)");
    void *ws = nullptr;
    if (need > 0 && (e = oeq::noalloc_scratch(&ws)) != hipSuccess)
        return fail(OEQ_ERR_HIP, std::string("scratch address: ") + hipGetErrorString(e));
    return oeq_tp_conv_bwd(plan, N, E, rowptr, src, x, Y, W, g, gx, gY, gW, mode, ws,
                           ws ? oeq::kNoAllocScratchBytes : 0, stream);
}

oeq_status oeq_tp_conv_dbwd(const oeq_plan *plan, int64_t N, int64_t E, const int32_t *rowptr, const int32_t *src,
                            const void *x, const void *Y, const void *W, const void *g, const void *ggx,
                            const void *ggY, const void *ggW, void *dx, void *dY, void *dW, void *dg,
                            oeq_bwd_mode mode, void *workspace, size_t workspace_bytes, void *stream) {
    oeq_status st = check_graph(plan, N, E, rowptr, src);
    if (st != OEQ_OK) return st;
    if (mode != OEQ_BWD_ATOMIC && mode != OEQ_BWD_DETERMINISTIC) return fail(OEQ_ERR_INVALID_ARG, "unknown mode");
    if (E > 0 && (!x || !Y || !W || !g)) return fail(OEQ_ERR_INVALID_ARG, "x, Y, W or grad_out is NULL");
    oeq_plan *p = const_cast<oeq_plan *>(plan);
    hipStream_t s = static_cast<hipStream_t>(stream);
    const int tm = (ggx ? 1 : 0) | (ggY ? 2 : 0) | (ggW ? 4 : 0);
    const int64_t PU = static_cast<int64_t>(p->paths.size()) * p->U;
    if (E == 0 || tm == 0) {
        if (dx && (st = fill_zero(p, dx, N * p->XD, s)) != OEQ_OK) return st;
        if (dY && (st = fill_zero(p, dY, E * p->YD, s)) != OEQ_OK) return st;
        if (dW && (st = fill_zero(p, dW, E * PU, s)) != OEQ_OK) return st;
        if (dg && (st = fill_zero(p, dg, N * p->OD, s)) != OEQ_OK) return st;
        return OEQ_OK;
    }
    if (tm == 1 && p->hvp_lds) {
        // the HVP from Y-contracted CG rows in LDS (d_x = 0 without a Y or W tangent)
        if (dx && (st = fill_zero(p, dx, N * p->XD, s)) != OEQ_OK) return st;
        if (!dY && !dW && !dg) return OEQ_OK;
        const int64_t NGB = static_cast<int64_t>(p->bwd_groups.size());
        const bool gyp = dY && NGB > 1;
        Workspace w;
        if ((st = ws_bind(p, N, E, false, gyp, workspace, workspace_bytes, &w)) != OEQ_OK) return st;
        int flags = (dW ? 1 : 0) | (dY ? 2 : 0) | (dg ? 4 : 0);
        void *dy_target = gyp ? w.gy_part : dY;
        int64_t gy_stride = gyp ? E * p->YD : 0;
        int n_nodes = static_cast<int>(N);
        void *args[] = {&rowptr, &src, &Y, &W, &g, &ggx, &dy_target, &dW, &dg, &flags, &gy_stride, &n_nodes};
        if ((st = launch(p, "oeq_hvp_lds", static_cast<unsigned>(N * NGB), bwd_block(p), s, args)) != OEQ_OK)
            return st;
        return gyp ? combine_parts(p, w.gy_part, static_cast<int>(NGB), dY, E * p->YD, s) : OEQ_OK;
    }
    // d_x = Bx(ggY,W,g) + Bx(Y,ggW,g) vanishes without a Y or W tangent
    const bool dx_live = dx && (tm & 6);
    const bool det = dx_live && mode == OEQ_BWD_DETERMINISTIC;
    auto spills = [&](const std::string &name, bool *yes) {
        hipFunction_t fn = nullptr;
        std::string why;
        const oeq_status r = oeq::get_kernel(*p, name.c_str(), &fn, &why);
        if (r != OEQ_OK) return fail(r, why);
        int scratch = 0;
        // a moderate spill costs less than a split. Measured on the fused kernels: 12, 144 and
        // 196 bytes per lane ran as fast as or faster than their splits (fp64 gg_x+gg_Y, large
        // gg_Y, fp64 gg_Y+gg_W); 276 bytes and up ran slower (large gg_x+gg_Y: 5.47 vs 4.85 ms)
        *yes = hipFuncGetAttribute(&scratch, HIP_FUNC_ATTRIBUTE_LOCAL_SIZE_BYTES, fn) == hipSuccess && scratch > 200;
        return OEQ_OK;
    };
    const std::string T = std::to_string(tm);
    // Passes of the split double backward (kernel name, which tangent bits it covers).
    //   d_W  = BW(gg_x,Y,g) + BW(x,gg_Y,g)                 oeq_dbwd_<tm&3>_1 (reads no weights)
    //   d_Y  = BY(gg_x,W,g) + BY(x,gg_W,g), d_x = Bx(gg_Y,W,g) + Bx(Y,gg_W,g)
    //        level 1: oeq_dbwd_<tm>_10 in one pass; level 2: one pass per tangent
    //   d_grad_out = f(gg_x,Y,W) + f(x,gg_Y,W) + f(x,Y,gg_W)  forward kernel, accumulating
    const bool single = tm == 1 || tm == 2 || tm == 4;
    const bool want_w = dW && (tm & 3), want_yx = (dY && (tm & 5)) || dx_live;
    std::vector<std::string> yx1;  // level-1 d_Y / d_x pass
    if (want_yx) yx1.push_back(single ? (tm == 1 ? "oeq_dbwd_1_2" : tm == 2 ? "oeq_dbwd_2_8" : "oeq_dbwd_4_10")
                                      : "oeq_dbwd_" + T + "_10");
    // One fused pass on the backward groups (oeq_dbwd_<t>) unless it spills; then the fused
    // pass on the finer double-backward groups (oeq_dbwd_<t>_d), where those differ; then
    // the split passes (on the double-backward groups).
    const bool two_sets = p->dbwd_groups != p->bwd_groups;
    std::string fused = "oeq_dbwd_" + T;
    int level = p->dbwd_split;  // 0 one fused pass, 1 or 2 split
    if (level < 0) {
        bool sp = false;
        if ((st = spills(fused, &sp)) != OEQ_OK) return st;
        level = 0;
        if (sp && two_sets) {
            fused = "oeq_dbwd_" + T + "_d";
            if ((st = spills(fused, &sp)) != OEQ_OK) return st;
        }
        if (sp) {
            level = 1;
            std::vector<std::string> k1 = yx1;
            if (want_w) k1.push_back("oeq_dbwd_" + std::to_string(tm & 3) + "_1");
            for (const auto &k : k1) {
                if ((st = spills(k, &sp)) != OEQ_OK) return st;
                if (sp) level = 2;
            }
        }
    }
    // Path groups of the kernels this call launches: oeq_dbwd_<t> is built on the backward
    // groups; oeq_dbwd_<t>_d and every split pass on the double-backward groups. The grid
    // must match: a kernel maps block b to receiver b / groups.
    auto kernel_groups = [&](const std::string &name) {
        const bool bwd_set = name.size() == 10 && name.compare(0, 9, "oeq_dbwd_") == 0;  // oeq_dbwd_<t>
        return static_cast<int64_t>(bwd_set ? p->bwd_groups.size() : p->dbwd_groups.size());
    };
    const int64_t NG = level == 0 ? kernel_groups(fused) : static_cast<int64_t>(p->dbwd_groups.size());
    const bool gyp = dY && NG > 1;
    const bool gxe = dx_live && needs_gxe(p);
    Workspace w;
    if ((st = ws_bind(p, N, E, det, gyp, workspace, workspace_bytes, &w, gxe)) != OEQ_OK) return st;
    if (dx && !dx_live && (st = fill_zero(p, dx, N * p->XD, s)) != OEQ_OK) return st;
    int dxmode = 0;
    void *dx_target = nullptr;
    if (dx_live && !det) {
        dx_target = gxe ? w.gxe : dx;  // rows of GXD values
        if ((st = fill_zero(p, dx_target, N * p->GXD, s)) != OEQ_OK) return st;
        dxmode = 1;
    } else if (det) {
        if ((st = sender_csr_into(N, E, src, w, s)) != OEQ_OK) return st;
        dxmode = 2;
        dx_target = w.h;
        if (p->x_unused && (st = fill_zero(p, w.h, E * p->GXD, s)) != OEQ_OK) return st;
    }
    if (!dxmode && !dY && !dW && !dg) return OEQ_OK;
    void *dy_target = gyp ? w.gy_part : dY;
    int64_t gy_stride = gyp ? E * p->YD : 0;
    const unsigned grid = static_cast<unsigned>(N * NG);
    auto pass = [&](const std::string &name, int flags) {
        // the kernel's own group count (the rule the kernel template applies); a grid of
        // another size would map blocks past the last receiver
        if (kernel_groups(name) != NG)
            return fail(OEQ_ERR_UNSUPPORTED, "internal: " + name + " is built for another path-group count");
        int n_nodes = static_cast<int>(N);
        void *args[] = {&rowptr, &src, &x, &Y, &W, &g, &ggx, &ggY, &ggW, &dx_target, &dy_target, &dW, &dg, &flags,
                        &gy_stride, &n_nodes};
        return launch(p, name.c_str(), grid, bwd_block(p), s, args);
    };
    if (level == 0) {
        const int flags = (dW ? 1 : 0) | (dY ? 2 : 0) | (dg ? 4 : 0) | (dxmode << 3);
        if ((st = pass(fused, flags)) != OEQ_OK) return st;
    } else {
        if (want_w && (st = pass("oeq_dbwd_" + std::to_string(tm & 3) + "_1", 1)) != OEQ_OK) return st;
        if (dW && !want_w && (st = fill_zero(p, dW, E * PU, s)) != OEQ_OK) return st;
        if (want_yx && (level == 1 || single)) {
            if ((st = pass(yx1[0], (dY && (tm & 5) ? 2 : 0) | (dxmode << 3))) != OEQ_OK) return st;
        } else if (want_yx) {
            bool wrote_dy = false, wrote_h = false;
            const struct {
                int bit;
                const char *name;
                bool y, x;
            } parts[] = {{1, "oeq_dbwd_1_2", true, false}, {2, "oeq_dbwd_2_8", false, true},
                         {4, "oeq_dbwd_4_10", true, true}};
            for (const auto &q : parts) {
                if (!(tm & q.bit)) continue;
                const bool py = dY && q.y;
                const int dm = q.x ? dxmode : 0;
                if (!py && !dm) continue;
                const int flags = (py ? 2 : 0) | (dm << 3) | (py && wrote_dy ? 64 : 0) | (dm == 2 && wrote_h ? 256 : 0);
                if ((st = pass(q.name, flags)) != OEQ_OK) return st;
                wrote_dy |= py;
                wrote_h |= dm == 2;
            }
        }
        if (dY && !(tm & 5) &&
            (st = fill_zero(p, dy_target, E * p->YD * (gyp ? NG : 1), s)) !=
                OEQ_OK)
            return st;
        if (dg) {
            int f = 0;
            if ((tm & 1) && (st = fwd_launch(p, N, rowptr, src, ggx, Y, W, dg, f, s)) != OEQ_OK) return st;
            f = tm & 1;
            if ((tm & 2) && (st = fwd_launch(p, N, rowptr, src, x, ggY, W, dg, f, s)) != OEQ_OK) return st;
            f = tm & 3 ? 1 : 0;
            if ((tm & 4) && (st = fwd_launch(p, N, rowptr, src, x, Y, ggW, dg, f, s)) != OEQ_OK) return st;
        }
    }
    if (dxmode == 2 && (st = det_finish(p, N, w, dx, s)) != OEQ_OK) return st;
    if (dxmode == 1 && (st = untranspose(p, N, dx_target, s)) != OEQ_OK) return st;
    if (dxmode == 1 && gxe && (st = fold_x(p, N, dx_target, dx, s)) != OEQ_OK) return st;
    return gyp ? combine_parts(p, w.gy_part, static_cast<int>(NG), dY, E * p->YD, s) : OEQ_OK;
}

}  // extern "C"
