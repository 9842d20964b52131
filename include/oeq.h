/*
 * oeq.h - C ABI of the fused channel-wise (UVU) Clebsch-Gordan tensor-product
 * graph convolution for AMD Instinct MI355X (gfx950).
 *
 * The operation ("Receiver-streaming convolutions for channel-wise UVU tensor
 * products", opening post; the CG tensor product and its fusion with graph
 * convolution as in the abstract of "An Efficient Sparse Kernel Generator for
 * O(3)-Equivariant Deep Networks"):
 *
 *   for every edge e = (s -> r) of a receiver-sorted graph, every path
 *   p = (x block i1 of degree l1, Y degree l2 -> output degree l3) and every
 *   channel u < U:
 *     out[r, blk(p), u, m3] += sum_{m1,m2} C_{l1 l2 l3}[m1,m2,m3]
 *                              * x[s, i1, u, m1] * Y[e, l2, m2] * W[e, p, u]
 *
 * C is the real-basis Clebsch-Gordan table (orthonormal, real spherical-harmonic
 * basis with the Condon-Shortley phase, m = -l..l, l=1 ordered (y, z, x), each
 * table signed so that its first non-zero entry in row-major (m1, m2, m3) order is
 * positive).  W carries every weight: there is no extra normalisation factor.
 *
 * Memory layouts (all row-major, element offsets computed in 64 bits):
 *   rowptr [N+1] int32   receiver CSR, rowptr[0] = 0, rowptr[N] = E, non-decreasing
 *   src    [E]   int32   sender of edge e; edge e belongs to receiver r when
 *                        rowptr[r] <= e < rowptr[r+1]
 *   x      [N, XD]       x block i at xoff_i (the widths mul*(2l+1) of the blocks
 *                        before it), element u*(2 l_i + 1) + (m + l_i); a block of
 *                        one channel holds (m + l_i) only
 *   Y      [E, YD]       Y block j (one channel) at yoff_j = the widths 2l+1 of the
 *                        blocks before it, element yoff_j + (m2 + l_j); for the
 *                        default Y (degrees 0..L) element l2*l2 + (m2 + l2)
 *   W      [E, P, U]
 *   out    [N, OD]       output block o at ooff_o, element u*(2 l_o + 1) + (m + l_o);
 *                        a block of one channel holds (m + l_o) only
 * Gradients use the layout of the tensor they belong to.
 *
 * Conventions shared by every entry point:
 *   - Every tensor is caller-allocated device memory, element type = the plan's
 *     dtype (float or double), naturally aligned.  The library never allocates
 *     device memory inside a compute call; scratch memory is the caller's
 *     workspace (see oeq_workspace_size).
 *   - Calls are asynchronous on `stream` (a hipStream_t; NULL = the default
 *     stream).  Outputs are overwritten, never accumulated into.
 *   - Arguments are checked on the host only (no device reads, no
 *     synchronisation).  Graph preconditions (CSR shape above, 0 <= src[e] < N)
 *     are the caller's responsibility and are not checked; violating them is
 *     undefined behaviour.  oeq_csr_check validates them synchronously.
 *   - Errors are reported as oeq_status codes, never by aborting;
 *     oeq_last_error() gives a per-thread message for the last failure.  Faults
 *     during kernel execution surface at the caller's next synchronisation.
 *   - A plan is immutable after creation and may be used from several threads
 *     and streams at once.
 *   - Supported: degrees l <= 3 for x, Y and outputs; U = the largest x
 *     multiplicity (1..1024), every x and output block with U channels or one;
 *     dtype float32 or float64.
 *
 * UVW products that reduce to this one ("Receiver-streaming convolutions ...",
 * maintainer replies: the streaming path also takes UVW convolutions reducible to
 * UVU).  Read here as a weight diagonal in (u, w) up to a broadcast or a sum: an x
 * block of one channel feeds every channel u (x[s, i1, 0, m1] in place of
 * x[s, i1, u, m1]), and an output block of one channel receives the sum over u
 * (out[r, blk, 0, m3] += the sum over u of the terms above).  Such plans run the
 * receiver-stationary passes; the sender-stationary passes and the passes that
 * form W in the kernel refuse them with OEQ_ERR_UNSUPPORTED.
 */
#ifndef OEQ_H
#define OEQ_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
    OEQ_OK = 0,
    OEQ_ERR_INVALID_ARG = 1, /* null pointer, negative size, bad enum        */
    OEQ_ERR_UNSUPPORTED = 2, /* l > 3, a multiplicity neither U nor 1, dtype */
    OEQ_ERR_WORKSPACE = 3,   /* workspace missing or smaller than required   */
    OEQ_ERR_HIP = 4,         /* a HIP runtime call or kernel launch failed   */
    OEQ_ERR_JIT = 5          /* runtime compilation of the kernels failed    */
} oeq_status;

typedef enum { OEQ_F32 = 0, OEQ_F64 = 1 } oeq_dtype;

/* How the x gradient is scattered to senders in the backward passes.
 * ATOMIC: hardware floating-point atomics (summation order varies run to run).
 * DETERMINISTIC: per-edge contributions are written to the workspace and
 * summed per sender in increasing edge id (bitwise repeatable). */
typedef enum { OEQ_BWD_ATOMIC = 0, OEQ_BWD_DETERMINISTIC = 1 } oeq_bwd_mode;

typedef struct {
    int32_t mul;    /* multiplicity (channels)                */
    int32_t l;      /* degree 0..3                            */
    int32_t parity; /* +1 even, -1 odd                        */
} oeq_irrep;

typedef struct {
    int32_t in1; /* index into the x irreps                              */
    int32_t in2; /* index into the Y irreps (default Y: the degree l2)   */
    int32_t out; /* index into the output irreps                         */
} oeq_path;

/* Irreps descriptor of one tensor product ("Receiver-streaming convolutions for
 * channel-wise UVU tensor products", maintainer replies: the convolution is one
 * interface over irreps descriptors of its inputs and outputs).  All arrays are
 * host memory, read during oeq_plan_create only. */
typedef struct {
    const oeq_irrep *x_irreps;   /* x blocks: U channels (the largest multiplicity) */
                                 /*   or one (broadcast against the U channels)     */
    int32_t n_x;
    const oeq_irrep *y_irreps;   /* Y blocks in row order, multiplicity 1 each, any */
    int32_t n_y;                 /*   degrees 0..3 in any order and either parity,  */
                                 /*   total width sum(2l+1) <= 16.  NULL: the       */
                                 /*   spherical harmonics 0..y_lmax, parity (-1)^l  */
    int32_t y_lmax;              /* used when y_irreps == NULL                      */
    const oeq_irrep *out_irreps; /* NULL: one output block of U channels per path,  */
                                 /*   in path order; given: U channels or one (the  */
                                 /*   sum over the channels) per block              */
    int32_t n_out;
    const oeq_path *paths;       /* NULL: enumerate every triangle-allowed path:    */
    int32_t n_paths;             /*   x blocks in order, then Y blocks in order,    */
                                 /*   l3 = |l1-l2|..min(l1+l2, lmax_out),           */
                                 /*   output parity p1 * pY                         */
    int32_t lmax_out;            /* used when paths == NULL                         */
    oeq_dtype dtype;
} oeq_tp_desc;

typedef struct oeq_plan oeq_plan; /* opaque, host-owned */

/* Builds the path list and the real-basis CG tables, emits the specialised HIP
 * kernels and compiles them for gfx950 (runtime compilation, cached on disk by a
 * hash of the generated source in $OEQ_CACHE_DIR, default: a "jitcache" folder
 * beside the library).  The kernels are specialised per descriptor when the
 * model is set up, as the CG kernel generator analyses each tensor product
 * before its kernels are built ("An Efficient Sparse Kernel Generator for
 * O(3)-Equivariant Deep Networks", abstract), and the streaming convolution is
 * its own template, chosen when the kernels are compiled at run time
 * ("Receiver-streaming convolutions ...", first maintainer reply).  The compile
 * runs in the helper program oeq_jitc beside the library (a child process with
 * this ROCm installation's compiler): compiled inside a process that had already
 * loaded another ROCm release's compiler library (a framework wheel that bundles
 * its own), the runtime compiler would use that release's LLVM, and on MI355X
 * its forward took 0.95 ms against 0.36 ms.  OEQ_JIT_IN_PROCESS=1, or a missing
 * or failing helper, compiles in the calling process instead.  Host-only;
 * the code object is loaded on a device at
 * the first compute call there.  *plan is set to NULL on failure.
 * Errors: OEQ_ERR_INVALID_ARG (NULL pointers, bad parity, a path outside the
 * triangle rule or with the wrong output parity), OEQ_ERR_UNSUPPORTED (degree
 * above 3, an x or output multiplicity other than U or 1, Y wider than 16, more
 * than 128 paths, an unknown dtype), OEQ_ERR_JIT (the runtime compiler failed). */
oeq_status oeq_plan_create(const oeq_tp_desc *desc, oeq_plan **plan);

/* As oeq_plan_create, but never runs the runtime compiler: returns OEQ_ERR_JIT
 * (with *plan = NULL) when the plan's code object is not in the cache (for
 * callers that must not compile, or compile ahead of time elsewhere). */
oeq_status oeq_plan_create_cached(const oeq_tp_desc *desc, oeq_plan **plan);
void oeq_plan_destroy(oeq_plan *plan);

/* Row widths of the tensors of the layouts above ("Receiver-streaming
 * convolutions ...", opening post: x per node, Y and W per edge, outputs per
 * receiver): x_dim = XD, y_dim = YD, out_dim = OD, w_per_edge = P*U.
 * Any output pointer may be NULL.  OEQ_ERR_INVALID_ARG for a NULL plan. */
oeq_status oeq_plan_dims(const oeq_plan *plan, int64_t *x_dim, int64_t *y_dim,
                         int64_t *out_dim, int64_t *n_paths, int64_t *w_per_edge);

/* Path k of the plan as (x block, l1, l2, l3, output block, output parity),
 * written to out6[6*k .. 6*k+5] for k < n_paths (host memory). */
oeq_status oeq_plan_paths(const oeq_plan *plan, int32_t *out6, int32_t capacity);

/* Identifier of the plan's compiled code object (hex hash of the generated
 * source and compile options), NUL-terminated into buf (host memory, at least
 * 17 bytes).  Lets measurements tie counter data to the exact kernels. */
oeq_status oeq_plan_code_key(const oeq_plan *plan, char *buf, size_t len);

/* The plan's real-basis CG table for (l1, l2, l3) as a dense fp64 array
 * [(2l1+1)(2l2+1)(2l3+1)] in host memory (the values the kernels use, before
 * rounding to the plan dtype).  Returns OEQ_ERR_INVALID_ARG outside the
 * triangle rule or l > 3. */
oeq_status oeq_cg_table(int32_t l1, int32_t l2, int32_t l3, double *out);

/* Workspace bytes a backward or double-backward call may need for `mode`
 * (per-group partial Y-gradients when the plan splits its paths over several
 * backward or double-backward groups, sized for the larger count; per-edge
 * x-gradient rows and the sender CSR for DETERMINISTIC: the materialised
 * per-edge tensor reduced in a fixed order of the deterministic fallback in
 * "Optimize UMA SO2 and Wigner inference kernels"); for ATOMIC with one-channel
 * x blocks, x-gradient rows of U channels in every block, whose channels the call
 * then sums into grad_x.  One size serves both
 * calls.  0 means no workspace is needed; the caller allocates it (the library
 * never allocates in a compute call).  OEQ_ERR_INVALID_ARG for a NULL plan or
 * output, negative sizes or an unknown mode. */
oeq_status oeq_workspace_size(const oeq_plan *plan, int64_t n_nodes, int64_t n_edges,
                              oeq_bwd_mode mode, size_t *bytes);

/* Forward: out = f(x, Y, W).  Receiver-stationary: one lane owns one
 * (receiver, channel), streams the receiver's edges and writes its output row
 * once, without atomics ("Receiver-streaming convolutions ...", opening post,
 * forward ownership).  Bitwise repeatable.  The forward takes no workspace, so it
 * always runs receiver-stationary; where oeq_plan_schedule prefers the
 * sender-stationary forward, oeq_tp_conv_fwd_sender runs it on a sender view. */
oeq_status oeq_tp_conv_fwd(const oeq_plan *plan, int64_t n_nodes, int64_t n_edges,
                           const int32_t *rowptr, const int32_t *src, const void *x,
                           const void *Y, const void *W, void *out, void *stream);

/* Vector-Jacobian product of <grad_out, f(x, Y, W)>:
 *   grad_W[e,p,u] = sum C x[s,u,m1] Y[e,m2] grad_out[r,u,m3]
 *   grad_Y[e,m2]  = sum_u sum_p sum C x[s,u,m1] W[e,p,u] grad_out[r,u,m3]
 *   grad_x[s,u,m1]= sum_{e: src[e]=s} sum_p sum C Y[e,m2] W[e,p,u] grad_out[r,u,m3]
 * Receiver-stationary and edge-streaming ("Receiver-streaming convolutions ...",
 * opening post, backward ownership): the waves of a workgroup take one receiver's
 * edges one at a time, lanes span channels, grad_W is written directly, grad_Y is
 * reduced across lanes, grad_x is scattered per `mode`.  Any of grad_x, grad_Y, grad_W may be NULL (not computed).
 * When the plan's data-movement model prefers the sender-stationary VJP
 * (oeq_plan_schedule; the choice is made once, at plan creation, as the
 * maintainers' reply in "Receiver-streaming convolutions ..." proposes), the call
 * builds the sender view of the graph in the workspace and runs
 * oeq_tp_conv_bwd_sender instead: no atomics, so every output is bitwise
 * repeatable in either mode.  Callers that keep a sender view across calls can
 * call oeq_tp_conv_bwd_sender directly and skip the view build.
 * `workspace` (256-byte aligned) must hold oeq_workspace_size(mode) bytes when
 * that size is not 0; a missing or small workspace gives OEQ_ERR_WORKSPACE. */
oeq_status oeq_tp_conv_bwd(const oeq_plan *plan, int64_t n_nodes, int64_t n_edges,
                           const int32_t *rowptr, const int32_t *src, const void *x,
                           const void *Y, const void *W, const void *grad_out,
                           void *grad_x, void *grad_Y, void *grad_W, oeq_bwd_mode mode,
                           void *workspace, size_t workspace_bytes, void *stream);

/* oeq_tp_conv_bwd without a workspace argument and without any allocation, for
 * callers that cannot allocate device memory: code under HIP graph capture, tight
 * serving loops, harnesses that forbid allocation.  Its scratch (the per-edge
 * x-gradient rows and the sender CSR of DETERMINISTIC mode, the per-group partial
 * Y-gradients of a plan with several backward groups, the ATOMIC x-gradient rows of
 * U channels per block of a plan with one-channel x blocks) lives in a file-scope device
 * array of 64 MiB that each device the library runs on holds until the process
 * ends; a call needing more returns OEQ_ERR_WORKSPACE with the size in
 * oeq_last_error(), before any device work.  The plan must already have run an
 * ordinary call on the current device (loading its kernels allocates), else
 * OEQ_ERR_INVALID_ARG.  Every call on a device shares that device's array:
 * calls that overlap on one device (several streams or threads at once) race
 * and must be ordered by the caller.  Results equal oeq_tp_conv_bwd's (bitwise
 * in DETERMINISTIC mode). */
oeq_status oeq_tp_conv_bwd_noalloc(const oeq_plan *plan, int64_t n_nodes, int64_t n_edges,
                                   const int32_t *rowptr, const int32_t *src, const void *x,
                                   const void *Y, const void *W, const void *grad_out,
                                   void *grad_x, void *grad_Y, void *grad_W, oeq_bwd_mode mode,
                                   void *stream);

/* Double backward: gradients of
 *   S = <gg_x, grad_x> + <gg_Y, grad_Y> + <gg_W, grad_W>
 * (grad_* the VJP above) with respect to x, Y, W and grad_out.  Since f is
 * linear in each of x, Y, W separately,
 *   d_grad_out = f(gg_x,Y,W) + f(x,gg_Y,W) + f(x,Y,gg_W)
 *   d_x = Bx(gg_Y,W,g) + Bx(Y,gg_W,g),   d_Y = BY(gg_x,W,g) + BY(x,gg_W,g),
 *   d_W = BW(gg_x,Y,g) + BW(x,gg_Y,g)
 * with Bx, BY, BW the three VJP components (the abstract of "An Efficient Sparse
 * Kernel Generator ..." names an identity for these higher derivatives without
 * printing it; this is the one used here).  A NULL tangent is zero; a NULL
 * output is not computed. */
oeq_status oeq_tp_conv_dbwd(const oeq_plan *plan, int64_t n_nodes, int64_t n_edges,
                            const int32_t *rowptr, const int32_t *src, const void *x,
                            const void *Y, const void *W, const void *grad_out,
                            const void *gg_x, const void *gg_Y, const void *gg_W,
                            void *d_x, void *d_Y, void *d_W, void *d_grad_out,
                            oeq_bwd_mode mode, void *workspace, size_t workspace_bytes,
                            void *stream);

/* Sender CSR of a receiver CSR (stable counting sort by sender): srowptr[N+1],
 * sperm[E] = edge ids grouped by sender, increasing within a sender.  Device
 * arrays; uses `workspace` of oeq_csr_workspace_size bytes; asynchronous. */
oeq_status oeq_csr_workspace_size(int64_t n_nodes, int64_t n_edges, size_t *bytes);
oeq_status oeq_sender_csr(int64_t n_nodes, int64_t n_edges, const int32_t *src,
                          int32_t *srowptr, int32_t *sperm, void *workspace,
                          size_t workspace_bytes, void *stream);

/* ---- Sender-stationary schedule ------------------------------------------
 * The maintainers' reply in "Receiver-streaming convolutions ..." proposes two
 * implementations of the convolution, "source stationary" and "destination
 * stationary", with the one that moves less data chosen at initialisation from
 * the input and output irreps.  The entry points above are destination
 * (receiver) stationary.  These are the source (sender) stationary pair: a
 * workgroup owns one sender, keeps its x row in registers and visits the
 * sender's out-edges through the sender view of the graph.
 *
 * oeq_plan_schedule reports the plan's choice and the per-edge, per-channel
 * costs of its model, in gathered elements (both schedules stream W and Y once;
 * one atomic add counts as 6 gathered elements, the ratio measured on MI355X):
 *   forward: receiver-stationary gathers x[s] (move_fwd[0] = x width per channel);
 *            sender-stationary adds into out[r] atomically (move_fwd[1] = 6 x
 *            output width per channel);
 *   VJP:     receiver-stationary gathers x[s] and adds into grad_x[s] atomically
 *            (move_bwd[0] = 7 x width); sender-stationary gathers grad_out[r]
 *            (move_bwd[1] = output width).
 * The smaller count wins (ties: receiver-stationary).  Each pointer may be NULL. */
typedef enum { OEQ_RECEIVER_STATIONARY = 0, OEQ_SENDER_STATIONARY = 1 } oeq_schedule;
oeq_status oeq_plan_schedule(const oeq_plan *plan, oeq_schedule *fwd, oeq_schedule *bwd,
                             double *move_fwd2, double *move_bwd2);

/* Sender view of a receiver CSR: oeq_sender_csr's srowptr[N+1] and sperm[E],
 * plus sdst[E] = the receiver of edge sperm[k].  Device arrays, built with
 * kernels only; `workspace` of oeq_csr_workspace_size bytes (256-byte aligned);
 * asynchronous.  A model whose graph is fixed builds it once. */
oeq_status oeq_sender_view(int64_t n_nodes, int64_t n_edges, const int32_t *rowptr,
                           const int32_t *src, int32_t *srowptr, int32_t *sperm,
                           int32_t *sdst, void *workspace, size_t workspace_bytes,
                           void *stream);

/* Forward, sender-stationary: out = f(x, Y, W) as oeq_tp_conv_fwd, with each
 * edge's message added into out[receiver] by floating-point atomics (so the
 * summation order varies run to run).  out is zeroed and reordered by the call
 * (two light kernels around the main one).  OEQ_ERR_UNSUPPORTED for a plan with a
 * one-channel x or output block. */
oeq_status oeq_tp_conv_fwd_sender(const oeq_plan *plan, int64_t n_nodes, int64_t n_edges,
                                  const int32_t *srowptr, const int32_t *sperm,
                                  const int32_t *sdst, const void *x, const void *Y,
                                  const void *W, void *out, void *stream);

/* VJP, sender-stationary: the gradients of oeq_tp_conv_bwd.  grad_out[r] is
 * gathered per edge; grad_W and grad_Y are per edge; grad_x of each sender is
 * accumulated in registers and stored once, without atomics, so every output is
 * bitwise repeatable.  Any gradient pointer may be NULL.  `workspace` must hold
 * oeq_workspace_size(plan, N, E, OEQ_BWD_ATOMIC) bytes when that size is not 0.
 * OEQ_ERR_UNSUPPORTED for a plan with a one-channel x or output block. */
oeq_status oeq_tp_conv_bwd_sender(const oeq_plan *plan, int64_t n_nodes, int64_t n_edges,
                                  const int32_t *srowptr, const int32_t *sperm,
                                  const int32_t *sdst, const void *x, const void *Y,
                                  const void *W, const void *grad_out, void *grad_x,
                                  void *grad_Y, void *grad_W, void *workspace,
                                  size_t workspace_bytes, void *stream);

/* ---- Y from edge vectors ---------------------------------------------------
 * The step before the tensor product: Y[e] = the real spherical harmonics of the
 * direction of the edge vector vec[e] = (x, y, z) (receiver-major edges are built
 * from atom positions; "Receiver-streaming convolutions ...", opening post), and
 * the gradient carried back from Y to the vectors.  Convention as for Y
 * everywhere in this library: the plan's Y blocks (each filled with the harmonics
 * of its degree), m = -l..l, degree 1 ordered (y, z, x), Condon-Shortley phase,
 * component normalisation (the squares of degree l sum to 2l+1).  The vector need
 * not be unit length; a zero vector gives Y_00 = 1, all other degrees 0, and a
 * zero gradient.  vec is [E, 3] in the plan's dtype.  Every entry point that
 * takes vectors returns OEQ_ERR_UNSUPPORTED for a plan with a Y block whose
 * parity is not (-1)^l (harmonics of a vector cannot fill it). */
oeq_status oeq_sph_harm(const oeq_plan *plan, int64_t n_edges, const void *vec, void *Y,
                        void *stream);

/* grad_vec[e] = sum_m grad_Y[e, m] dY[e, m] / dvec[e]  ([E, 3]). */
oeq_status oeq_sph_harm_bwd(const oeq_plan *plan, int64_t n_edges, const void *vec,
                            const void *grad_Y, void *grad_vec, void *stream);

/* Forward from edge vectors: out = f(x, Y(vec), W), with the harmonics evaluated
 * inside the forward kernel (no Y tensor is read or written).  Otherwise as
 * oeq_tp_conv_fwd. */
oeq_status oeq_tp_conv_fwd_vec(const oeq_plan *plan, int64_t n_nodes, int64_t n_edges,
                               const int32_t *rowptr, const int32_t *src, const void *x,
                               const void *vec, const void *W, void *out, void *stream);

/* VJP from edge vectors: grad_x, grad_W as oeq_tp_conv_bwd, and
 * grad_vec[e] = sum_m grad_Y[e,m] dY[e,m]/dvec[e] in place of grad_Y.  Runs
 * oeq_sph_harm into the workspace, the VJP, then oeq_sph_harm_bwd.  `workspace`
 * (256-byte aligned) must hold oeq_workspace_size_vec(mode) bytes. */
oeq_status oeq_workspace_size_vec(const oeq_plan *plan, int64_t n_nodes, int64_t n_edges,
                                  oeq_bwd_mode mode, size_t *bytes);
oeq_status oeq_tp_conv_bwd_vec(const oeq_plan *plan, int64_t n_nodes, int64_t n_edges,
                               const int32_t *rowptr, const int32_t *src, const void *x,
                               const void *vec, const void *W, const void *grad_out,
                               void *grad_x, void *grad_vec, void *grad_W, oeq_bwd_mode mode,
                               void *workspace, size_t workspace_bytes, void *stream);

/* ---- Y from atom positions ---------------------------------------------------
 * The same with the edges' vectors formed from atom positions pos[N, 3] (plan
 * dtype): vec[e] = pos[src[e]] - pos[r] for edge e of receiver row r, the
 * neighbour's position relative to the central atom of a neighbour list
 * ("Receiver-streaming convolutions ...", opening post: receiver-major edges come
 * from the neighbour lists of atom positions).  The VJP returns, in place of
 * grad_Y, the gradient of <grad_out, f> with respect to the positions:
 *   grad_pos[n] = sum_{e: src[e] = n} grad_vec[e] - sum_{e in row n} grad_vec[e],
 * scattered with floating-point atomics (ATOMIC) or summed per node in a fixed
 * order, out-edges in increasing edge id then the node's own row
 * (DETERMINISTIC: bitwise repeatable).  The forward evaluates the harmonics
 * inside the kernel; the VJP forms vectors and Y into the workspace, runs the VJP,
 * then the harmonic gradient and the scatter.  A self-loop has a zero vector and
 * contributes nothing to grad_pos.  `workspace` (256-byte aligned) must hold
 * oeq_workspace_size_pos(mode) bytes.  Errors as for the vector entry points. */
oeq_status oeq_tp_conv_fwd_pos(const oeq_plan *plan, int64_t n_nodes, int64_t n_edges,
                               const int32_t *rowptr, const int32_t *src, const void *x,
                               const void *pos, const void *W, void *out, void *stream);
oeq_status oeq_workspace_size_pos(const oeq_plan *plan, int64_t n_nodes, int64_t n_edges,
                                  oeq_bwd_mode mode, size_t *bytes);
oeq_status oeq_tp_conv_bwd_pos(const oeq_plan *plan, int64_t n_nodes, int64_t n_edges,
                               const int32_t *rowptr, const int32_t *src, const void *x,
                               const void *pos, const void *W, const void *grad_out,
                               void *grad_x, void *grad_pos, void *grad_W, oeq_bwd_mode mode,
                               void *workspace, size_t workspace_bytes, void *stream);

/* ---- Radial weights from edge lengths ---------------------------------------
 * The pages realise W outside the convolution, and fusing its realisation would be
 * a new operation ("Receiver-streaming convolutions ...", maintainer replies).  They
 * give no specification; these entry points compute this stated one (the shape
 * used by MACE-style potentials):
 *   r = |vec[e]|, d = r / r_cut
 *   u(d)   = 1 - 28 d^6 + 48 d^7 - 21 d^8 for d < 1, else 0       (polynomial cutoff, p = 6)
 *   B_n(r) = sqrt(2 / r_cut) sin(n pi r / r_cut) / r * u(d), n = 1..8  (limit n pi / r_cut at r = 0)
 *   h      = silu(B W1 / sqrt(8))                                 W1 [8, hidden]
 *   W[e]   = h W2 / sqrt(hidden), viewed as [P, U]                W2 [hidden, P*U]
 * The two dense products (and the three of the backward) run on the matrix
 * cores.  vec [E, 3], W1, W2 and W in the plan's dtype; hidden in 1..1024.
 * `workspace` (256-byte aligned) of oeq_radial_workspace_size bytes. */
oeq_status oeq_radial_workspace_size(const oeq_plan *plan, int64_t n_edges, int32_t hidden,
                                     size_t *bytes);
oeq_status oeq_radial_fwd(const oeq_plan *plan, int64_t n_edges, const void *vec, double r_cut,
                          int32_t hidden, const void *W1, const void *W2, void *W,
                          void *workspace, size_t workspace_bytes, void *stream);

/* Gradients of <grad_W, W(vec, W1, W2)> with respect to vec ([E, 3]), W1 and W2
 * (sums over the edges, added in a fixed order: bitwise repeatable).  Any of
 * grad_vec, grad_W1, grad_W2 may be NULL. */
oeq_status oeq_radial_bwd(const oeq_plan *plan, int64_t n_edges, const void *vec, double r_cut,
                          int32_t hidden, const void *W1, const void *W2, const void *grad_W,
                          void *grad_vec, void *grad_W1, void *grad_W2, void *workspace,
                          size_t workspace_bytes, void *stream);

/* Forward with the radial weights formed inside the convolution kernel (no W
 * tensor is written or read): out = f(x, Y, W) with W = oeq_radial_fwd(vec, r_cut,
 * 8, W1, W2), for a hidden width of exactly 8 (W1 [8, 8], W2 [8, P*U]).  Each lane
 * keeps its slice of W2 in registers and forms W[e] from the edge's 8 hidden
 * values.  `workspace` of oeq_radial_workspace_size(plan, E, 8) bytes holds the
 * basis and the hidden values.  OEQ_ERR_UNSUPPORTED for a plan with a one-channel
 * x or output block. */
oeq_status oeq_tp_conv_fwd_radial(const oeq_plan *plan, int64_t n_nodes, int64_t n_edges,
                                  const int32_t *rowptr, const int32_t *src, const void *x,
                                  const void *Y, const void *vec, double r_cut, const void *W1,
                                  const void *W2, void *out, void *workspace,
                                  size_t workspace_bytes, void *stream);

/* VJP of oeq_tp_conv_fwd_radial (hidden width 8, W formed in the kernel): grad_x
 * and grad_Y as oeq_tp_conv_bwd, and, in place of grad_W, the gradients of the
 * radial network: grad_vec [E, 3], grad_W1 [8, 8], grad_W2 [8, P*U].  Per edge the
 * kernel contracts its W gradient with W2 into the 8 hidden-value gradients
 * (reduced over lanes and waves like grad_Y) and accumulates h (x) gW into a
 * per-receiver W2-gradient row; the rows are summed over receivers in order, so
 * grad_W2 and grad_W1 are bitwise repeatable.  Any output may be NULL.  Needs Y
 * degrees up to at least 2.  `workspace` of oeq_workspace_size_radial bytes.
 * OEQ_ERR_UNSUPPORTED for a plan with a one-channel x or output block. */
oeq_status oeq_workspace_size_radial(const oeq_plan *plan, int64_t n_nodes, int64_t n_edges,
                                     oeq_bwd_mode mode, size_t *bytes);
oeq_status oeq_tp_conv_bwd_radial(const oeq_plan *plan, int64_t n_nodes, int64_t n_edges,
                                  const int32_t *rowptr, const int32_t *src, const void *x,
                                  const void *Y, const void *vec, double r_cut, const void *W1,
                                  const void *W2, const void *grad_out, void *grad_x,
                                  void *grad_Y, void *grad_vec, void *grad_W1, void *grad_W2,
                                  oeq_bwd_mode mode, void *workspace, size_t workspace_bytes,
                                  void *stream);

/* Synchronously validates a receiver CSR on the device (rowptr monotone,
 * rowptr[0] = 0, rowptr[N] = E, 0 <= src < N).  Test helper: synchronises. */
oeq_status oeq_csr_check(int64_t n_nodes, int64_t n_edges, const int32_t *rowptr,
                         const int32_t *src, void *stream);

const char *oeq_status_string(oeq_status status);
const char *oeq_last_error(void);

#ifdef __cplusplus
}
#endif
#endif /* OEQ_H */
