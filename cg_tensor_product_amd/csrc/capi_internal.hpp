// Internal helpers shared by the C-ABI source files (not part of the ABI):
// error reporting, argument checks, kernel launches, workspace layouts and the
// dense-product launcher.
#pragma once

#include <algorithm>
#include <cmath>
#include <cstdint>
#include <cstdlib>
#include <cstring>
#include <limits>
#include <string>

#include "csr.hpp"
#include "planner.hpp"

namespace oeq {
namespace capi {

inline thread_local std::string g_last_error;

inline oeq_status fail(oeq_status st, const std::string &msg) {
    g_last_error = msg;
    return st;
}

constexpr size_t kAlign = 256;
inline size_t up(size_t v) { return (v + kAlign - 1) / kAlign * kAlign; }
inline size_t esize(const oeq_plan *p) { return p->dtype == OEQ_F64 ? 8 : 4; }

// Threads per workgroup: one wave per (64-channel chunk, path group).
inline unsigned fwd_block(const oeq_plan *p) { return static_cast<unsigned>(p->uch * p->fwd_groups.size() * 64); }
inline unsigned bwd_block(const oeq_plan *p) { return static_cast<unsigned>(p->uch * 64); }
// oeq_fwd: one workgroup per receiver, or with fwd_xcd one per (receiver, chunk) in an order
// that keeps each chunk on the same XCDs (the kernel maps the workgroup id back)
inline unsigned fwd_wg(const oeq_plan *p) {
    return static_cast<unsigned>((p->fwd_xcd ? 1 : p->uch) * p->fwd_groups.size() * 64);
}
inline unsigned fwd_grid(const oeq_plan *p, int64_t N) {
    if (!p->fwd_xcd) return static_cast<unsigned>(N);
    if (8 % p->uch == 0) {
        const int64_t per = 8 / p->uch;  // XCDs of one chunk
        return static_cast<unsigned>(8 * ((N + per - 1) / per));
    }
    return static_cast<unsigned>(N * p->uch);
}

inline oeq_status check_graph(const oeq_plan *p, int64_t N, int64_t E, const int32_t *rowptr, const int32_t *src) {
    if (!p) return fail(OEQ_ERR_INVALID_ARG, "plan is NULL");
    if (N < 0 || E < 0) return fail(OEQ_ERR_INVALID_ARG, "negative node or edge count");
    if (N >= std::numeric_limits<int32_t>::max() || E >= std::numeric_limits<int32_t>::max())
        return fail(OEQ_ERR_UNSUPPORTED, "node and edge counts must fit the int32 CSR");
    if (N == 0 && E != 0) return fail(OEQ_ERR_INVALID_ARG, "edges without nodes");
    const int64_t groups = static_cast<int64_t>(std::max({p->bwd_groups.size(), p->dbwd_groups.size(), p->rad_groups.size()}));
    if (N * std::max<int64_t>(fwd_block(p), static_cast<int64_t>(bwd_block(p)) * groups) >=
        (int64_t(1) << 32))
        return fail(OEQ_ERR_UNSUPPORTED, "too many nodes for one launch");
    if (N > 0 && !rowptr) return fail(OEQ_ERR_INVALID_ARG, "rowptr is NULL");
    if (E > 0 && !src) return fail(OEQ_ERR_INVALID_ARG, "src is NULL");
    return OEQ_OK;
}

inline oeq_status launch(oeq_plan *p, const char *name, unsigned grid, unsigned block, hipStream_t stream, void **args) {
    if (grid == 0) return OEQ_OK;
    hipFunction_t fn = nullptr;
    std::string why;
    oeq_status st = oeq::get_kernel(*p, name, &fn, &why);
    if (st != OEQ_OK) return fail(st, why);
    const hipError_t e = hipModuleLaunchKernel(fn, grid, 1, 1, block, 1, 1, 0, stream, args, nullptr);
    if (e != hipSuccess) return fail(OEQ_ERR_HIP, std::string("launch ") + name + ": " + hipGetErrorString(e));
    return OEQ_OK;
}

inline oeq_status fill_zero(oeq_plan *p, void *ptr, int64_t n, hipStream_t stream) {
    if (n <= 0) return OEQ_OK;
    int64_t blocks = (n + 255) / 256;
    if (blocks > 65536) blocks = 65536;
    void *args[] = {&ptr, &n};
    return launch(p, "oeq_fill_zero", static_cast<unsigned>(blocks), 256, stream, args);
}

// Reorders atomically accumulated x-gradient rows from m-major to u-major blocks.
inline oeq_status untranspose(oeq_plan *p, int64_t N, void *gx, hipStream_t stream) {
    if (!p->xt) return OEQ_OK;
    void *args[] = {&gx};
    return launch(p, "oeq_x_untranspose", static_cast<unsigned>(N), 256, stream, args);
}

// Caller-provided scratch, carved in 256-byte aligned pieces:
//   gy_part  partial Y-gradient rows of each backward path group (several groups only)
//   h, srowptr, sperm, csr_scratch   deterministic x-gradient (per-edge rows of GXD values,
//            sender CSR)
//   gxe      x-gradient rows of GXD values (plans with one-channel x blocks: the channels
//            are summed into the caller's rows afterwards)
struct Workspace {
    void *gy_part = nullptr;
    void *h = nullptr;
    int32_t *srowptr = nullptr, *sperm = nullptr;
    void *csr_scratch = nullptr;
    void *gxe = nullptr;
    size_t bytes = 0;
};

// Whether an atomic x-gradient of this plan goes through GXD-wide rows in the workspace.
inline bool needs_gxe(const oeq_plan *p) { return p->GXD != p->XD; }

// Plans with one-channel x or output blocks run the receiver-stationary passes only.
inline oeq_status check_channelwise(const oeq_plan *p, const char *what) {
    if (p && (p->bcast_x || p->sum_out))
        return fail(OEQ_ERR_UNSUPPORTED, std::string(what) + " needs U channels in every x and output block");
    return OEQ_OK;
}

// per-group Y-gradient partials are sized for the larger of the VJP's and the double
// backward's group counts, so that one workspace size serves both
inline size_t gy_groups(const oeq_plan *p) { return std::max(p->bwd_groups.size(), p->dbwd_groups.size()); }

inline oeq_status ws_layout(const oeq_plan *p, int64_t N, int64_t E, bool det, bool gy_part, char *base, Workspace *w,
                            bool gxe = false) {
    size_t off = 0;
    if (gxe) {
        w->gxe = base + off;
        off += up(static_cast<size_t>(N) * static_cast<size_t>(p->GXD) * esize(p));
    }
    if (gy_part) {
        w->gy_part = base + off;
        off += up(gy_groups(p) * static_cast<size_t>(E) * p->YD * esize(p));
    }
    if (det) {
        size_t csr_bytes = 0;
        const hipError_t e = oeq::sender_csr_workspace(N, E, &csr_bytes);
        if (e != hipSuccess) return fail(OEQ_ERR_HIP, std::string("sender CSR workspace: ") + hipGetErrorString(e));
        w->h = base + off;
        off += up(static_cast<size_t>(E) * static_cast<size_t>(p->GXD) * esize(p));
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

// Workspace of a VJP that the plan's data-movement model sends to the sender-stationary
// pass: the sender view (srowptr[N+1], sperm[E], sdst[E]) and its build scratch, then the
// pass's own partial Y-gradient rows (several backward groups).
struct SenderWs {
    size_t srowptr = 0, sperm = 0, sdst = 0, csr = 0, vjp = 0, bytes = 0;
};

inline oeq_status sender_ws_layout(const oeq_plan *p, int64_t N, int64_t E, SenderWs *w) {
    size_t csr_bytes = 0;
    const hipError_t e = oeq::sender_csr_workspace(N, E, &csr_bytes);
    if (e != hipSuccess) return fail(OEQ_ERR_HIP, std::string("sender CSR workspace: ") + hipGetErrorString(e));
    const size_t ne = static_cast<size_t>(E > 0 ? E : 1);
    size_t off = 0;
    w->srowptr = off;
    off += up(sizeof(int32_t) * static_cast<size_t>(N + 1));
    w->sperm = off;
    off += up(sizeof(int32_t) * ne);
    w->sdst = off;
    off += up(sizeof(int32_t) * ne);
    w->csr = off;
    off += up(csr_bytes);
    w->vjp = off;
    if (p->bwd_groups.size() > 1) off += up(gy_groups(p) * static_cast<size_t>(E) * p->YD * esize(p));
    w->bytes = off;
    return OEQ_OK;
}

// Whether oeq_tp_conv_bwd takes the sender-stationary pass (the model's choice; a graph
// without edges needs no pass).
inline bool bwd_by_sender(const oeq_plan *p, int64_t E) { return p->sched_bwd == 1 && E > 0; }

// Bytes of workspace an oeq_tp_conv_bwd call binds for these requested outputs.
inline oeq_status bwd_ws_bytes(const oeq_plan *p, int64_t N, int64_t E, oeq_bwd_mode mode, bool gx, bool gY,
                               size_t *bytes) {
    *bytes = 0;
    if (E <= 0) return OEQ_OK;
    if (bwd_by_sender(p, E)) {
        SenderWs sw;
        oeq_status st = sender_ws_layout(p, N, E, &sw);
        if (st == OEQ_OK) *bytes = sw.bytes;
        return st;
    }
    Workspace w;
    oeq_status st = ws_layout(p, N, E, gx && mode == OEQ_BWD_DETERMINISTIC, gY && p->bwd_groups.size() > 1, nullptr, &w,
                              gx && needs_gxe(p));
    if (st == OEQ_OK) *bytes = w.bytes;
    return st;
}

// Bytes of workspace oeq_tp_conv_bwd may bind for a mode, whatever outputs are requested:
// the receiver-stationary layout, or the sender view when the plan routes the VJP there.
inline oeq_status vjp_ws_bytes(const oeq_plan *p, int64_t N, int64_t E, oeq_bwd_mode mode, size_t *bytes) {
    Workspace w;
    oeq_status st = ws_layout(p, N, E, mode == OEQ_BWD_DETERMINISTIC, gy_groups(p) > 1, nullptr, &w, needs_gxe(p));
    if (st != OEQ_OK) return st;
    *bytes = w.bytes;
    if (bwd_by_sender(p, E)) {
        SenderWs sw;
        if ((st = sender_ws_layout(p, N, E, &sw)) != OEQ_OK) return st;
        *bytes = std::max(*bytes, sw.bytes);
    }
    return OEQ_OK;
}

// Carves the workspace a call needs; fails before any device work if it is
// missing, misaligned or too small.
inline oeq_status ws_bind(const oeq_plan *p, int64_t N, int64_t E, bool det, bool gy_part, void *workspace,
                   size_t ws_bytes, Workspace *w, bool gxe = false) {
    if (!det && !gy_part && !gxe) return OEQ_OK;
    if (!workspace) return fail(OEQ_ERR_WORKSPACE, "this call needs a workspace (see oeq_workspace_size)");
    if (reinterpret_cast<uintptr_t>(workspace) % kAlign)
        return fail(OEQ_ERR_WORKSPACE, "workspace must be 256-byte aligned");
    oeq_status st = ws_layout(p, N, E, det, gy_part, static_cast<char *>(workspace), w, gxe);
    if (st != OEQ_OK) return st;
    if (ws_bytes < w->bytes) return fail(OEQ_ERR_WORKSPACE, "workspace smaller than oeq_workspace_size");
    return OEQ_OK;
}

inline oeq_status sender_csr_into(int64_t N, int64_t E, const int32_t *src, const Workspace &w, hipStream_t stream) {
    const hipError_t e = oeq::sender_csr(N, E, src, w.srowptr, w.sperm, w.csr_scratch, stream);
    if (e != hipSuccess) return fail(OEQ_ERR_HIP, std::string("sender CSR: ") + hipGetErrorString(e));
    return OEQ_OK;
}

inline oeq_status fold_x(oeq_plan *p, int64_t N, const void *gxe, void *gx, hipStream_t stream);

// x-gradient by per-edge rows (already written to w.h) summed per sender; with one-channel
// x blocks into the GXD-wide rows w.gxe, whose channels are then summed into gx.
inline oeq_status det_finish(oeq_plan *p, int64_t N, const Workspace &w, void *gx, hipStream_t stream) {
    void *h = w.h;
    int32_t *srp = w.srowptr, *spm = w.sperm;
    int n = static_cast<int>(N);
    void *dst = needs_gxe(p) ? w.gxe : gx;
    void *args[] = {&srp, &spm, &h, &dst, &n};
    oeq_status st = launch(p, "oeq_sender_sum", static_cast<unsigned>(N), 256, stream, args);
    if (st != OEQ_OK || !needs_gxe(p)) return st;
    return fold_x(p, N, w.gxe, gx, stream);
}

// The caller's x-gradient rows from the GXD-wide rows of the atomic passes.
inline oeq_status fold_x(oeq_plan *p, int64_t N, const void *gxe, void *gx, hipStream_t stream) {
    int64_t n = N * p->XD;
    if (n <= 0) return OEQ_OK;
    const int64_t blocks = std::min<int64_t>((n + 255) / 256, 65536);
    void *args[] = {&gxe, &gx, &n};
    return launch(p, "oeq_fold_x", static_cast<unsigned>(blocks), 256, stream, args);
}

inline oeq_status gy_combine(oeq_plan *p, const Workspace &w, void *gY, int64_t E, hipStream_t stream) {
    int64_t n = E * p->YD;
    if (n <= 0) return OEQ_OK;
    int64_t blocks = (n + 255) / 256;
    if (blocks > 65536) blocks = 65536;
    void *part = w.gy_part;
    void *args[] = {&part, &gY, &n};
    return launch(p, "oeq_gy_combine", static_cast<unsigned>(blocks), 256, stream, args);
}

// flags bit0: add into out instead of overwriting it
inline oeq_status fwd_launch(oeq_plan *p, int64_t N, const int32_t *rowptr, const int32_t *src, const void *x, const void *Y,
                      const void *W, void *out, int flags, hipStream_t s) {
    int n_nodes = static_cast<int>(N);
    void *args[] = {&rowptr, &src, &x, &Y, &W, &out, &flags, &n_nodes};
    return launch(p, "oeq_fwd", fwd_grid(p, N), fwd_wg(p), s, args);
}

// Grid-stride launch of a per-edge kernel (vec, a, b, n) over E edges.
inline oeq_status edge_launch(oeq_plan *p, const char *name, int64_t E, void **args, hipStream_t stream) {
    int64_t blocks = (E + 255) / 256;
    if (blocks > 65536) blocks = 65536;
    return launch(p, name, static_cast<unsigned>(blocks), 256, stream, args);
}

// C[M,N] (ldc) = the sum of `rows` partial [M, N] matrices stored densely in `part`, added in
// row order: in two stages when there are many (chunks of 32 rows in parallel into `scratch`,
// ceil(rows/32) x M x N elements, then the chunk sums).
inline oeq_status ordered_sum(oeq_plan *p, void *part, int rows, int M, int N, void *C, int64_t ldc, void *scratch,
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
inline int choose_splits(int64_t K, int64_t tiles) {
    const int64_t want = (2048 + tiles - 1) / std::max<int64_t>(tiles, 1);
    return static_cast<int>(std::max<int64_t>(1, std::min<int64_t>(want, K / 256)));
}

// C[M,N] = alpha op(A)[M,K] op(B)[K,N] on the matrix cores (oeq_gemm).  With
// splits > 1 the K range is cut into that many pieces whose tiles go to `part`
// ([splits, M, N]) and are then added in order into C.
inline oeq_status gemm(oeq_plan *p, int M, int N, int K, const void *A, int64_t lda, bool ta, const void *B, int64_t ldb,
                bool tb, void *C, int64_t ldc, double alpha, int splits, void *part, hipStream_t s) {
    if (M <= 0 || N <= 0) return OEQ_OK;
    int kchunk = std::max(K, 1);
    if (splits > 1) {
        kchunk = ((K + splits - 1) / splits + 15) / 16 * 16;
        splits = (K + kchunk - 1) / kchunk;
    }
    if (splits < 1) splits = 1;

    void *dst = splits > 1 ? part : C;
    int64_t ldd = splits > 1 ? N : ldc;
    int64_t stride = static_cast<int64_t>(M) * N;
    float af = static_cast<float>(alpha);
    void *ap = p->dtype == OEQ_F64 ? static_cast<void *>(&alpha) : static_cast<void *>(&af);
    if (ta && tb) return fail(OEQ_ERR_UNSUPPORTED, "both operands transposed");
    void *args[] = {&M, &N, &K, &A, &lda, &B, &ldb, &dst, &ldd, &stride, &kchunk, ap};
    // 128-wide tile sides where the matrix fills them; fp64 keeps 64 x 64 (its 128-wide tiles
    // hold one wave per SIMD and ran slower, as did 128 rows over a 64-row matrix)
    const bool wide = p->dtype == OEQ_F32;
    const int bm = wide && M >= 128 ? 128 : 64, bn = wide && N >= 128 ? 128 : 64;
    const std::string kname = "oeq_gemm_" + std::to_string(bm) + "x" + std::to_string(bn) + "_" + (ta ? "1" : "0") +
                              (tb ? "1" : "0");
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
inline size_t gemm_part_elems(int M, int N, int splits) {
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
inline int64_t gemm_tiles(const oeq_plan *p, int M, int N) {
    const bool wide = p->dtype == OEQ_F32;
    const int bm = wide && M >= 128 ? 128 : 64, bn = wide && N >= 128 ? 128 : 64;
    return static_cast<int64_t>((M + bm - 1) / bm) * ((N + bn - 1) / bn);
}
constexpr int kFusedHidden = 8;  // hidden width of the forward that forms W in the kernel

inline RadialWs radial_layout(const oeq_plan *p, int64_t E, int H) {
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

inline oeq_status radial_check(const oeq_plan *p, int64_t E, double r_cut, int H, const void *vec, const void *W1,
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
inline oeq_status radial_hidden(oeq_plan *p, int64_t E, const void *vec, double r_cut, int H, const void *W1, char *ws,
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



// Workspace of the radial VJP: the radial pieces (width 8), the VJP's sender CSR and
// per-edge x-gradient rows (deterministic mode), the per-group partial gY and dh rows
// (several radial groups) and the per-receiver dW2 partials [N, 8, P*U].
struct RadVjpWs {
    RadialWs rad;
    Workspace conv;
    size_t conv_off = 0, gyp = 0, dhp = 0, w2p = 0, w2s = 0, wbuf = 0, gwbuf = 0, bytes = 0;
};

inline oeq_status radvjp_layout(const oeq_plan *p, int64_t N, int64_t E, bool det, char *base, RadVjpWs *w) {
    const size_t es = esize(p), PU = p->paths.size() * static_cast<size_t>(p->U), G = p->rad_groups.size();
    w->rad = radial_layout(p, E, kFusedHidden);
    size_t off = w->rad.bytes;
    w->conv_off = off;
    if (p->rad_compose) {  // the convolution VJP's own workspace, then W and its gradient
        oeq_status st = vjp_ws_bytes(p, N, E, det ? OEQ_BWD_DETERMINISTIC : OEQ_BWD_ATOMIC, &w->conv.bytes);
        if (st != OEQ_OK) return st;
        off += up(w->conv.bytes);
        w->wbuf = off;
        off += up(static_cast<size_t>(E) * PU * es);
        w->gwbuf = off;
        off += up(static_cast<size_t>(E) * PU * es);
        w->bytes = off;
        return OEQ_OK;
    }
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

inline oeq_status combine_parts(oeq_plan *p, void *part, int groups, void *out, int64_t n, hipStream_t s) {
    if (n <= 0) return OEQ_OK;
    int64_t blocks = std::min<int64_t>((n + 255) / 256, 65536);
    void *args[] = {&part, &groups, &out, &n};
    return launch(p, "oeq_part_combine", static_cast<unsigned>(blocks), 256, s, args);
}

}  // namespace capi
}  // namespace oeq
