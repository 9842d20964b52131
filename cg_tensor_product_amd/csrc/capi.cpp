// C ABI entry points: argument checks (host only, no device reads, no
// synchronisation), workspace carving and stream-ordered kernel launches.
#include <algorithm>
#include <cmath>
#include <cstdlib>
#include <cstring>
#include <limits>
#include <string>

#include "csr.hpp"
#include "planner.hpp"

namespace {

thread_local std::string g_last_error;

oeq_status fail(oeq_status st, const std::string &msg) {
    g_last_error = msg;
    return st;
}

constexpr size_t kAlign = 256;
size_t up(size_t v) { return (v + kAlign - 1) / kAlign * kAlign; }
size_t esize(const oeq_plan *p) { return p->dtype == OEQ_F64 ? 8 : 4; }

// Threads per workgroup: one wave per (64-channel chunk, path group).
unsigned fwd_block(const oeq_plan *p) { return static_cast<unsigned>(p->uch * p->fwd_groups.size() * 64); }
unsigned bwd_block(const oeq_plan *p) { return static_cast<unsigned>(p->uch * 64); }

oeq_status check_graph(const oeq_plan *p, int64_t N, int64_t E, const int32_t *rowptr, const int32_t *src) {
    if (!p) return fail(OEQ_ERR_INVALID_ARG, "plan is NULL");
    if (N < 0 || E < 0) return fail(OEQ_ERR_INVALID_ARG, "negative node or edge count");
    if (N >= std::numeric_limits<int32_t>::max() || E >= std::numeric_limits<int32_t>::max())
        return fail(OEQ_ERR_UNSUPPORTED, "node and edge counts must fit the int32 CSR");
    if (N == 0 && E != 0) return fail(OEQ_ERR_INVALID_ARG, "edges without nodes");
    if (N * std::max<int64_t>(fwd_block(p), static_cast<int64_t>(bwd_block(p)) * p->bwd_groups.size()) >=
        (int64_t(1) << 32))
        return fail(OEQ_ERR_UNSUPPORTED, "too many nodes for one launch");
    if (N > 0 && !rowptr) return fail(OEQ_ERR_INVALID_ARG, "rowptr is NULL");
    if (E > 0 && !src) return fail(OEQ_ERR_INVALID_ARG, "src is NULL");
    return OEQ_OK;
}

oeq_status launch(oeq_plan *p, const char *name, unsigned grid, unsigned block, hipStream_t stream, void **args) {
    if (grid == 0) return OEQ_OK;
    hipFunction_t fn = nullptr;
    std::string why;
    oeq_status st = oeq::get_kernel(*p, name, &fn, &why);
    if (st != OEQ_OK) return fail(st, why);
    const hipError_t e = hipModuleLaunchKernel(fn, grid, 1, 1, block, 1, 1, 0, stream, args, nullptr);
    if (e != hipSuccess) return fail(OEQ_ERR_HIP, std::string("launch ") + name + ": " + hipGetErrorString(e));
    return OEQ_OK;
}

oeq_status fill_zero(oeq_plan *p, void *ptr, int64_t n, hipStream_t stream) {
    if (n <= 0) return OEQ_OK;
    int64_t blocks = (n + 255) / 256;
    if (blocks > 65536) blocks = 65536;
    void *args[] = {&ptr, &n};
    return launch(p, "oeq_fill_zero", static_cast<unsigned>(blocks), 256, stream, args);
}

// Reorders atomically accumulated x-gradient rows from m-major to u-major blocks.
oeq_status untranspose(oeq_plan *p, int64_t N, void *gx, hipStream_t stream) {
    if (!p->xt) return OEQ_OK;
    void *args[] = {&gx};
    return launch(p, "oeq_x_untranspose", static_cast<unsigned>(N), 256, stream, args);
}

// Caller-provided scratch, carved in 256-byte aligned pieces:
//   gy_part  partial Y-gradient rows of each backward path group (several groups only)
//   h, srowptr, sperm, csr_scratch   deterministic x-gradient (per-edge rows, sender CSR)
struct Workspace {
    void *gy_part = nullptr;
    void *h = nullptr;
    int32_t *srowptr = nullptr, *sperm = nullptr;
    void *csr_scratch = nullptr;
    size_t bytes = 0;
};

oeq_status ws_layout(const oeq_plan *p, int64_t N, int64_t E, bool det, bool gy_part, char *base, Workspace *w) {
    size_t off = 0;
    if (gy_part) {
        w->gy_part = base + off;
        off += up(p->bwd_groups.size() * static_cast<size_t>(E) * p->YD * esize(p));
    }
    if (det) {
        size_t csr_bytes = 0;
        const hipError_t e = oeq::sender_csr_workspace(N, E, &csr_bytes);
        if (e != hipSuccess) return fail(OEQ_ERR_HIP, std::string("sender CSR workspace: ") + hipGetErrorString(e));
        w->h = base + off;
        off += up(static_cast<size_t>(E) * static_cast<size_t>(p->XD) * esize(p));
        w->srowptr = reinterpret_cast<int32_t *>(base + off);
        off += up(sizeof(int32_t) * static_cast<size_t>(N + 1));
        w->sperm = reinterpret_cast<int32_t *>(base + off);
        off += up(sizeof(int32_t) * static_cast<size_t>(E > 0 ? E : 1));
        w->csr_scratch = base + off;
        off += up(csr_bytes);
    }
    w->bytes = off;
    return OEQ_OK;
}

// Carves the workspace a call needs; fails before any device work if it is
// missing, misaligned or too small.
oeq_status ws_bind(const oeq_plan *p, int64_t N, int64_t E, bool det, bool gy_part, void *workspace,
                   size_t ws_bytes, Workspace *w) {
    if (!det && !gy_part) return OEQ_OK;
    if (!workspace) return fail(OEQ_ERR_WORKSPACE, "this call needs a workspace (see oeq_workspace_size)");
    if (reinterpret_cast<uintptr_t>(workspace) % kAlign)
        return fail(OEQ_ERR_WORKSPACE, "workspace must be 256-byte aligned");
    oeq_status st = ws_layout(p, N, E, det, gy_part, static_cast<char *>(workspace), w);
    if (st != OEQ_OK) return st;
    if (ws_bytes < w->bytes) return fail(OEQ_ERR_WORKSPACE, "workspace smaller than oeq_workspace_size");
    return OEQ_OK;
}

oeq_status sender_csr_into(int64_t N, int64_t E, const int32_t *src, const Workspace &w, hipStream_t stream) {
    const hipError_t e = oeq::sender_csr(N, E, src, w.srowptr, w.sperm, w.csr_scratch, stream);
    if (e != hipSuccess) return fail(OEQ_ERR_HIP, std::string("sender CSR: ") + hipGetErrorString(e));
    return OEQ_OK;
}

// x-gradient by per-edge rows (already written to w.h) summed per sender.
oeq_status det_finish(oeq_plan *p, int64_t N, const Workspace &w, void *gx, hipStream_t stream) {
    void *h = w.h;
    int32_t *srp = w.srowptr, *spm = w.sperm;
    int n = static_cast<int>(N);
    void *args[] = {&srp, &spm, &h, &gx, &n};
    return launch(p, "oeq_sender_sum", static_cast<unsigned>(N), 256, stream, args);
}

oeq_status gy_combine(oeq_plan *p, const Workspace &w, void *gY, int64_t E, hipStream_t stream) {
    int64_t n = E * p->YD;
    if (n <= 0) return OEQ_OK;
    int64_t blocks = (n + 255) / 256;
    if (blocks > 65536) blocks = 65536;
    void *part = w.gy_part;
    void *args[] = {&part, &gY, &n};
    return launch(p, "oeq_gy_combine", static_cast<unsigned>(blocks), 256, stream, args);
}

// flags bit0: add into out instead of overwriting it
oeq_status fwd_launch(oeq_plan *p, int64_t N, const int32_t *rowptr, const int32_t *src, const void *x, const void *Y,
                      const void *W, void *out, int flags, hipStream_t s) {
    void *args[] = {&rowptr, &src, &x, &Y, &W, &out, &flags};
    return launch(p, "oeq_fwd", static_cast<unsigned>(N), fwd_block(p), s, args);
}

// Grid-stride launch of a per-edge kernel (vec, a, b, n) over E edges.
oeq_status edge_launch(oeq_plan *p, const char *name, int64_t E, void **args, hipStream_t stream) {
    int64_t blocks = (E + 255) / 256;
    if (blocks > 65536) blocks = 65536;
    return launch(p, name, static_cast<unsigned>(blocks), 256, stream, args);
}

// C[M,N] (ldc) = the sum of `rows` partial [M, N] matrices stored densely in `part`, added in
// row order: in two stages when there are many (chunks of 32 rows in parallel into `scratch`,
// ceil(rows/32) x M x N elements, then the chunk sums).
oeq_status ordered_sum(oeq_plan *p, void *part, int rows, int M, int N, void *C, int64_t ldc, void *scratch,
                       hipStream_t s) {
    int64_t n = static_cast<int64_t>(M) * N;
    if (n <= 0 || rows <= 0) return OEQ_OK;
    oeq_status st;
    if (rows > 32 && scratch) {
        const int chunks = (rows + 31) / 32;
        void *args[] = {&part, &rows, &n, &scratch};
        hipFunction_t fn = nullptr;
        std::string why;
        if ((st = oeq::get_kernel(*p, "oeq_sum_row_chunks", &fn, &why)) != OEQ_OK) return fail(st, why);
        const hipError_t e = hipModuleLaunchKernel(fn, static_cast<unsigned>((n + 255) / 256),
                                                   static_cast<unsigned>(chunks), 1, 256, 1, 1, 0, s, args, nullptr);
        if (e != hipSuccess) return fail(OEQ_ERR_HIP, std::string("launch oeq_sum_row_chunks: ") + hipGetErrorString(e));
        part = scratch;
        rows = chunks;
    }
    int64_t blocks = std::min<int64_t>((n + 255) / 256, 65536);
    void *rargs[] = {&part, &rows, &n, &M, &N, &C, &ldc};
    return launch(p, "oeq_gemm_reduce", static_cast<unsigned>(blocks), 256, s, rargs);
}

// Splits of K for a product whose output has `tiles` workgroup tiles: enough workgroups
// to fill the chip, at least 256 K values each.
int choose_splits(int64_t K, int64_t tiles) {
    const int64_t want = (2048 + tiles - 1) / std::max<int64_t>(tiles, 1);
    return static_cast<int>(std::max<int64_t>(1, std::min<int64_t>(want, K / 256)));
}

// C[M,N] = alpha op(A)[M,K] op(B)[K,N] on the matrix cores (oeq_gemm).  With
// splits > 1 the K range is cut into that many pieces whose tiles go to `part`
// ([splits, M, N]) and are then added in order into C.
oeq_status gemm(oeq_plan *p, int M, int N, int K, const void *A, int64_t lda, bool ta, const void *B, int64_t ldb,
                bool tb, void *C, int64_t ldc, double alpha, int splits, void *part, hipStream_t s) {
    if (M <= 0 || N <= 0) return OEQ_OK;
    int kchunk = std::max(K, 1);
    if (splits > 1) {
        kchunk = ((K + splits - 1) / splits + 15) / 16 * 16;
        splits = (K + kchunk - 1) / kchunk;
    }
    if (splits < 1) splits = 1;
    int ta_i = ta ? 1 : 0, tb_i = tb ? 1 : 0;
    void *dst = splits > 1 ? part : C;
    int64_t ldd = splits > 1 ? N : ldc;
    int64_t stride = static_cast<int64_t>(M) * N;
    float af = static_cast<float>(alpha);
    void *ap = p->dtype == OEQ_F64 ? static_cast<void *>(&alpha) : static_cast<void *>(&af);
    void *args[] = {&M, &N, &K, &A, &lda, &ta_i, &B, &ldb, &tb_i, &dst, &ldd, &stride, &kchunk, ap};
    // 128-wide tile sides where the matrix fills them; fp64 keeps 64 x 64 (its 128-wide tiles
    // hold one wave per SIMD and ran slower, as did 128 rows over a 64-row matrix)
    const bool wide = p->dtype == OEQ_F32;
    const int bm = wide && M >= 128 ? 128 : 64, bn = wide && N >= 128 ? 128 : 64;
    const std::string kname = "oeq_gemm_" + std::to_string(bm) + "x" + std::to_string(bn);
    const char *name = kname.c_str();
    hipFunction_t fn = nullptr;
    std::string why;
    oeq_status st = oeq::get_kernel(*p, name, &fn, &why);
    if (st != OEQ_OK) return fail(st, why);
    const hipError_t e = hipModuleLaunchKernel(fn, static_cast<unsigned>((N + bn - 1) / bn),
                                               static_cast<unsigned>((M + bm - 1) / bm), static_cast<unsigned>(splits),
                                               256, 1, 1, 0, s, args, nullptr);
    if (e != hipSuccess) return fail(OEQ_ERR_HIP, std::string("launch ") + name + ": " + hipGetErrorString(e));
    if (splits == 1) return OEQ_OK;
    // the chunk sums go after the partial tiles (the caller sizes `part` with gemm_part_elems)
    void *scratch = static_cast<char *>(part) + static_cast<size_t>(splits) * stride * esize(p);
    return ordered_sum(p, part, splits, M, N, C, ldc, scratch, s);
}

// Elements of `part` a gemm() call with this many splits needs.
size_t gemm_part_elems(int M, int N, int splits) {
    const size_t n = static_cast<size_t>(M) * N;
    return splits > 1 ? n * (splits + (splits + 31) / 32) : 0;
}

// Workspace of the radial-weight passes: B [E,8], h [E,H], dh [E,H], dB [E,8], then the
// split-K partials of the two products summed over edges.
struct RadialWs {
    size_t B = 0, h = 0, dh = 0, dB = 0, pW2 = 0, pW1 = 0, bytes = 0;
    int splitsW2 = 1, splitsW1 = 1;
};
constexpr int kRadialNB = 8;

// workgroup tiles of gemm() for an M x N output (its tile choice)
int64_t gemm_tiles(const oeq_plan *p, int M, int N) {
    const bool wide = p->dtype == OEQ_F32;
    const int bm = wide && M >= 128 ? 128 : 64, bn = wide && N >= 128 ? 128 : 64;
    return static_cast<int64_t>((M + bm - 1) / bm) * ((N + bn - 1) / bn);
}
constexpr int kFusedHidden = 8;  // hidden width of the forward that forms W in the kernel

RadialWs radial_layout(const oeq_plan *p, int64_t E, int H) {
    RadialWs w;
    const size_t es = esize(p), PU = p->paths.size() * static_cast<size_t>(p->U);
    w.splitsW2 = choose_splits(E, gemm_tiles(p, H, static_cast<int>(PU)));
    w.splitsW1 = choose_splits(E, gemm_tiles(p, kRadialNB, H));
    size_t off = 0;
    w.B = off;
    off += up(static_cast<size_t>(E) * kRadialNB * es);
    w.h = off;
    off += up(static_cast<size_t>(E) * H * es);
    w.dh = off;
    off += up(static_cast<size_t>(E) * H * es);
    w.dB = off;
    off += up(static_cast<size_t>(E) * kRadialNB * es);
    w.pW2 = off;
    off += up(gemm_part_elems(H, static_cast<int>(PU), w.splitsW2) * es);
    w.pW1 = off;
    off += up(gemm_part_elems(kRadialNB, H, w.splitsW1) * es);
    w.bytes = off;
    return w;
}

oeq_status radial_check(const oeq_plan *p, int64_t E, double r_cut, int H, const void *vec, const void *W1,
                        const void *W2, void *workspace, size_t bytes, RadialWs *w) {
    if (!p) return fail(OEQ_ERR_INVALID_ARG, "plan is NULL");
    if (E < 0) return fail(OEQ_ERR_INVALID_ARG, "negative edge count");
    if (E >= std::numeric_limits<int32_t>::max()) return fail(OEQ_ERR_UNSUPPORTED, "edge count must fit int32");
    if (H < 1 || H > 1024) return fail(OEQ_ERR_UNSUPPORTED, "hidden width must be 1..1024");
    if (!(r_cut > 0.0)) return fail(OEQ_ERR_INVALID_ARG, "r_cut must be positive");
    if (E > 0 && (!vec || !W1 || !W2)) return fail(OEQ_ERR_INVALID_ARG, "vec, W1 or W2 is NULL");
    *w = radial_layout(p, E, H);
    if (E > 0 && (!workspace || bytes < w->bytes)) return fail(OEQ_ERR_WORKSPACE, "workspace too small");
    if (reinterpret_cast<uintptr_t>(workspace) % kAlign)
        return fail(OEQ_ERR_WORKSPACE, "workspace must be 256-byte aligned");
    return OEQ_OK;
}

// B and h of every edge into the workspace
oeq_status radial_hidden(oeq_plan *p, int64_t E, const void *vec, double r_cut, int H, const void *W1, char *ws,
                         const RadialWs &w, hipStream_t s) {
    void *Bp = ws + w.B, *hp = ws + w.h;
    float rcf = static_cast<float>(r_cut);
    void *rc = p->dtype == OEQ_F64 ? static_cast<void *>(&r_cut) : static_cast<void *>(&rcf);
    void *bargs[] = {&vec, rc, &Bp, &E};
    oeq_status st = edge_launch(p, "oeq_radial_basis", E, bargs, s);
    if (st != OEQ_OK) return st;
    void *hargs[] = {&Bp, &W1, &H, &hp, &E};
    return edge_launch(p, "oeq_radial_hidden", E * H, hargs, s);
}

}  // namespace

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

oeq_status oeq_plan_create(const oeq_tp_desc *desc, oeq_plan **plan) {
    if (!plan) return fail(OEQ_ERR_INVALID_ARG, "plan output pointer is NULL");
    *plan = nullptr;
    oeq_plan *p = new oeq_plan();
    std::string why;
    oeq_status st = oeq::plan_build(desc, p, &why);
    if (st == OEQ_OK) {
        p->source = oeq::emit_source(*p);
        st = oeq::jit_compile(*p, &why);
    }
    if (st != OEQ_OK) {
        delete p;
        return fail(st, why);
    }
    *plan = p;
    return OEQ_OK;
}

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

oeq_status oeq_plan_schedule(const oeq_plan *p, oeq_schedule *fwd, oeq_schedule *bwd, double *move_fwd2,
                             double *move_bwd2) {
    if (!p) return fail(OEQ_ERR_INVALID_ARG, "plan is NULL");
    if (fwd) *fwd = p->sched_fwd ? OEQ_SENDER_STATIONARY : OEQ_RECEIVER_STATIONARY;
    if (bwd) *bwd = p->sched_bwd ? OEQ_SENDER_STATIONARY : OEQ_RECEIVER_STATIONARY;
    if (move_fwd2) std::memcpy(move_fwd2, p->move_fwd, sizeof p->move_fwd);
    if (move_bwd2) std::memcpy(move_bwd2, p->move_bwd, sizeof p->move_bwd);
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
    Workspace w;
    oeq_status st = ws_layout(p, n_nodes, n_edges, mode == OEQ_BWD_DETERMINISTIC, p->bwd_groups.size() > 1,
                              nullptr, &w);
    if (st != OEQ_OK) return st;
    *bytes = w.bytes;
    return OEQ_OK;
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
    const bool det = gx && mode == OEQ_BWD_DETERMINISTIC;
    const bool gyp = gY && p->bwd_groups.size() > 1;
    Workspace w;
    if ((st = ws_bind(p, N, E, det, gyp, workspace, workspace_bytes, &w)) != OEQ_OK) return st;
    int flags = (gW ? 1 : 0) | (gY ? 2 : 0);
    void *gy_target = gyp ? w.gy_part : gY;
    int64_t gy_stride = gyp ? E * p->YD : 0;
    const unsigned grid = static_cast<unsigned>(N * static_cast<int64_t>(p->bwd_groups.size()));
    const unsigned block = bwd_block(p);
    if (!gx) {
        void *args[] = {&rowptr, &src, &x, &Y, &W, &g, &gx, &gy_target, &gW, &flags, &gy_stride};
        st = launch(p, "oeq_bwd_nogx", grid, block, s, args);
    } else if (mode == OEQ_BWD_ATOMIC) {
        if ((st = fill_zero(p, gx, N * p->XD, s)) != OEQ_OK) return st;
        void *args[] = {&rowptr, &src, &x, &Y, &W, &g, &gx, &gy_target, &gW, &flags, &gy_stride};
        if ((st = launch(p, "oeq_bwd_atomic", grid, block, s, args)) != OEQ_OK) return st;
        st = untranspose(p, N, gx, s);
    } else {
        if ((st = sender_csr_into(N, E, src, w, s)) != OEQ_OK) return st;
        void *h = w.h;
        // an x block that feeds no path is never written into the per-edge rows
        if (p->x_unused && (st = fill_zero(p, h, E * p->XD, s)) != OEQ_OK) return st;
        void *args[] = {&rowptr, &src, &x, &Y, &W, &g, &h, &gy_target, &gW, &flags, &gy_stride};
        if ((st = launch(p, "oeq_bwd_rows", grid, block, s, args)) != OEQ_OK) return st;
        st = det_finish(p, N, w, gx, s);
    }
    if (st != OEQ_OK) return st;
    return gyp ? gy_combine(p, w, gY, E, s) : OEQ_OK;
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
    // d_x = Bx(ggY,W,g) + Bx(Y,ggW,g) vanishes without a Y or W tangent
    const bool dx_live = dx && (tm & 6);
    const bool det = dx_live && mode == OEQ_BWD_DETERMINISTIC;
    const bool gyp = dY && p->bwd_groups.size() > 1;
    Workspace w;
    if ((st = ws_bind(p, N, E, det, gyp, workspace, workspace_bytes, &w)) != OEQ_OK) return st;
    if (dx && !dx_live && (st = fill_zero(p, dx, N * p->XD, s)) != OEQ_OK) return st;
    int dxmode = 0;
    void *dx_target = nullptr;
    if (dx_live && !det) {
        if ((st = fill_zero(p, dx, N * p->XD, s)) != OEQ_OK) return st;
        dxmode = 1;
        dx_target = dx;
    } else if (det) {
        if ((st = sender_csr_into(N, E, src, w, s)) != OEQ_OK) return st;
        dxmode = 2;
        dx_target = w.h;
        if (p->x_unused && (st = fill_zero(p, w.h, E * p->XD, s)) != OEQ_OK) return st;
    }
    if (!dxmode && !dY && !dW && !dg) return OEQ_OK;
    void *dy_target = gyp ? w.gy_part : dY;
    int64_t gy_stride = gyp ? E * p->YD : 0;
    const unsigned grid = static_cast<unsigned>(N * static_cast<int64_t>(p->bwd_groups.size()));
    auto pass = [&](const std::string &name, int flags) {
        void *args[] = {&rowptr, &src, &x, &Y, &W, &g, &ggx, &ggY, &ggW, &dx_target, &dy_target, &dW, &dg, &flags,
                        &gy_stride};
        return launch(p, name.c_str(), grid, bwd_block(p), s, args);
    };
    auto spills = [&](const std::string &name, bool *yes) {
        hipFunction_t fn = nullptr;
        std::string why;
        const oeq_status r = oeq::get_kernel(*p, name.c_str(), &fn, &why);
        if (r != OEQ_OK) return fail(r, why);
        int scratch = 0;
        *yes = hipFuncGetAttribute(&scratch, HIP_FUNC_ATTRIBUTE_LOCAL_SIZE_BYTES, fn) == hipSuccess && scratch > 0;
        return OEQ_OK;
    };
    const std::string T = std::to_string(tm);
    // Passes of the split double backward (kernel name, which tangent bits it covers).
    //   d_W  = BW(gg_x,Y,g) + BW(x,gg_Y,g)                 oeq_dbwd_<tm&3>_1 (reads no weights)
    //   d_Y  = BY(gg_x,W,g) + BY(x,gg_W,g), d_x = Bx(gg_Y,W,g) + Bx(Y,gg_W,g)
    //        level 1: oeq_dbwd_<tm>_10 in one pass; level 2: one pass per tangent
    //   d_grad_out = f(gg_x,Y,W) + f(x,gg_Y,W) + f(x,Y,gg_W)  forward kernel, accumulating
    const bool single = tm == 1 || tm == 2 || tm == 4;
    const bool want_w = dW && (tm & 3), want_yx = (dY && (tm & 5)) || dxmode;
    std::vector<std::string> yx1;  // level-1 d_Y / d_x pass
    if (want_yx) yx1.push_back(single ? (tm == 1 ? "oeq_dbwd_1_2" : tm == 2 ? "oeq_dbwd_2_8" : "oeq_dbwd_4_10")
                                      : "oeq_dbwd_" + T + "_10");
    int level = p->dbwd_split;  // 0 one fused pass, 1 or 2 split
    if (level < 0) {
        bool sp = false;
        if ((st = spills("oeq_dbwd_" + T, &sp)) != OEQ_OK) return st;
        level = 0;
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
    if (level == 0) {
        const int flags = (dW ? 1 : 0) | (dY ? 2 : 0) | (dg ? 4 : 0) | (dxmode << 3);
        if ((st = pass("oeq_dbwd_" + T, flags)) != OEQ_OK) return st;
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
            (st = fill_zero(p, dy_target, E * p->YD * (gyp ? static_cast<int64_t>(p->bwd_groups.size()) : 1), s)) !=
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
    if (dxmode == 1 && (st = untranspose(p, N, dx, s)) != OEQ_OK) return st;
    return gyp ? gy_combine(p, w, dY, E, s) : OEQ_OK;
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
    if (E > 0 && !sdst) return fail(OEQ_ERR_INVALID_ARG, "sdst is NULL");
    if (N > 0 && !out) return fail(OEQ_ERR_INVALID_ARG, "out is NULL");
    if (E > 0 && (!x || !Y || !W)) return fail(OEQ_ERR_INVALID_ARG, "x, Y or W is NULL");
    oeq_plan *p = const_cast<oeq_plan *>(plan);
    hipStream_t s = static_cast<hipStream_t>(stream);
    if ((st = fill_zero(p, out, N * p->OD, s)) != OEQ_OK || E == 0) return st;
    void *args[] = {&srowptr, &sperm, &sdst, &x, &Y, &W, &out};
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
    void *args[] = {&srowptr, &sperm, &sdst, &x, &Y, &W, &g, &gx, &gy_target, &gW, &flags, &gy_stride};
    if ((st = launch(p, "oeq_bwd_sender", grid, bwd_block(p), s, args)) != OEQ_OK) return st;
    return gyp ? gy_combine(p, w, gY, E, s) : OEQ_OK;
}

oeq_status oeq_sph_harm(const oeq_plan *plan, int64_t E, const void *vec, void *Y, void *stream) {
    if (!plan) return fail(OEQ_ERR_INVALID_ARG, "plan is NULL");
    if (E < 0) return fail(OEQ_ERR_INVALID_ARG, "negative edge count");
    if (E == 0) return OEQ_OK;
    if (!vec || !Y) return fail(OEQ_ERR_INVALID_ARG, "vec or Y is NULL");
    oeq_plan *p = const_cast<oeq_plan *>(plan);
    void *args[] = {&vec, &Y, &E};
    return edge_launch(p, "oeq_sph_harm", E, args, static_cast<hipStream_t>(stream));
}

oeq_status oeq_sph_harm_bwd(const oeq_plan *plan, int64_t E, const void *vec, const void *gY, void *gvec,
                            void *stream) {
    if (!plan) return fail(OEQ_ERR_INVALID_ARG, "plan is NULL");
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
    if (N > 0 && !out) return fail(OEQ_ERR_INVALID_ARG, "out is NULL");
    if (E > 0 && (!x || !vec || !W)) return fail(OEQ_ERR_INVALID_ARG, "x, vec or W is NULL");
    oeq_plan *p = const_cast<oeq_plan *>(plan);
    void *args[] = {&rowptr, &src, &x, &vec, &W, &out};
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
    void *args[] = {&rowptr, &src, &x, &Y, &hid, &W2, &out};
    return launch(p, "oeq_fwd_radial", static_cast<unsigned>(N), fwd_block(p), s, args);
}

}  // extern "C"

namespace {

// Workspace of the radial VJP: the radial pieces (width 8), the VJP's sender CSR and
// per-edge x-gradient rows (deterministic mode), the per-group partial gY and dh rows
// (several radial groups) and the per-receiver dW2 partials [N, 8, P*U].
struct RadVjpWs {
    RadialWs rad;
    Workspace conv;
    size_t conv_off = 0, gyp = 0, dhp = 0, w2p = 0, w2s = 0, bytes = 0;
};

oeq_status radvjp_layout(const oeq_plan *p, int64_t N, int64_t E, bool det, char *base, RadVjpWs *w) {
    const size_t es = esize(p), PU = p->paths.size() * static_cast<size_t>(p->U), G = p->rad_groups.size();
    w->rad = radial_layout(p, E, kFusedHidden);
    size_t off = w->rad.bytes;
    w->conv_off = off;
    oeq_status st = ws_layout(p, N, E, det, false, base ? base + off : nullptr, &w->conv);
    if (st != OEQ_OK) return st;
    off += up(w->conv.bytes);
    w->gyp = off;
    if (G > 1) off += up(G * static_cast<size_t>(E) * p->YD * es);
    w->dhp = off;
    if (G > 1) off += up(G * static_cast<size_t>(E) * kFusedHidden * es);
    w->w2p = off;
    off += up(static_cast<size_t>(N) * kFusedHidden * PU * es);
    w->w2s = off;  // chunk sums of those rows
    off += up(static_cast<size_t>((N + 31) / 32) * kFusedHidden * PU * es);
    w->bytes = off;
    return OEQ_OK;
}

oeq_status combine_parts(oeq_plan *p, void *part, int groups, void *out, int64_t n, hipStream_t s) {
    if (n <= 0) return OEQ_OK;
    int64_t blocks = std::min<int64_t>((n + 255) / 256, 65536);
    void *args[] = {&part, &groups, &out, &n};
    return launch(p, "oeq_part_combine", static_cast<unsigned>(blocks), 256, s, args);
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
    int flags = (gW2 ? 1 : 0) | (gY ? 2 : 0) | (want_dh ? 4 : 0);
    void *hid = ws + w.rad.h, *dh = ws + w.rad.dh, *w2p = ws + w.w2p;
    void *gy_target = G > 1 ? ws + w.gyp : gY, *dh_target = G > 1 ? ws + w.dhp : dh;
    int64_t gy_stride = G > 1 ? E * p->YD : 0, dh_stride = G > 1 ? E * H : 0;
    const unsigned grid = static_cast<unsigned>(N * static_cast<int64_t>(G));
    const unsigned block = bwd_block(p);
    if (!gx) {
        void *args[] = {&rowptr, &src, &x, &Y, &hid, &W2, &g, &gx, &gy_target, &dh_target, &w2p, &flags, &gy_stride,
                        &dh_stride};
        if ((st = launch(p, "oeq_bwd_radial_nogx", grid, block, s, args)) != OEQ_OK) return st;
    } else if (!det) {
        if ((st = fill_zero(p, gx, N * p->XD, s)) != OEQ_OK) return st;
        void *args[] = {&rowptr, &src, &x, &Y, &hid, &W2, &g, &gx, &gy_target, &dh_target, &w2p, &flags, &gy_stride,
                        &dh_stride};
        if ((st = launch(p, "oeq_bwd_radial_atomic", grid, block, s, args)) != OEQ_OK) return st;
        if ((st = untranspose(p, N, gx, s)) != OEQ_OK) return st;
    } else {
        if ((st = sender_csr_into(N, E, src, w.conv, s)) != OEQ_OK) return st;
        void *hrows = w.conv.h;
        // each group writes the x blocks of its own paths; a block no path uses stays zero
        if (p->x_unused && (st = fill_zero(p, hrows, E * p->XD, s)) != OEQ_OK) return st;
        void *args[] = {&rowptr, &src, &x, &Y, &hid, &W2, &g, &hrows, &gy_target, &dh_target, &w2p, &flags,
                        &gy_stride, &dh_stride};
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
    if (!want_dh) return OEQ_OK;
    // the rest of the radial backward from dh: dpre, gW1 = B^T dpre / sqrt(8), dB, grad_vec
    void *Bp = ws + w.rad.B;
    const int Ei = static_cast<int>(E);
    const double s8 = 1.0 / std::sqrt(double(kRadialNB));
    void *dargs[] = {&Bp, &W1, const_cast<int *>(&H), &dh, &E};
    if ((st = edge_launch(p, "oeq_radial_dpre", E * H, dargs, s)) != OEQ_OK) return st;
    if (gW1 && (st = gemm(p, kRadialNB, H, Ei, Bp, kRadialNB, true, dh, H, false, gW1, H, s8, w.rad.splitsW1,
                          ws + w.rad.pW1, s)) != OEQ_OK)
        return st;
    if (!gvec) return OEQ_OK;
    void *dB = ws + w.rad.dB;
    if ((st = gemm(p, Ei, kRadialNB, H, dh, H, false, W1, H, true, dB, kRadialNB, s8, 1, nullptr, s)) != OEQ_OK)
        return st;
    float rcf = static_cast<float>(r_cut);
    void *rc = p->dtype == OEQ_F64 ? static_cast<void *>(&r_cut) : static_cast<void *>(&rcf);
    void *gargs[] = {&vec, rc, &dB, &gvec, &E};
    return edge_launch(p, "oeq_radial_gvec", E, gargs, s);
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
