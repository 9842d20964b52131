// Double backward.

// ---------------------------------------------------------------------------
// Double backward.  TM: which tangents are present (1 gg_x, 2 gg_Y, 4 gg_W).
//   d_grad_out = f(ggx,Y,W) + f(x,ggY,W) + f(x,Y,ggW)      (receiver-local)
//   d_W = BW(ggx,Y,g) + BW(x,ggY,g),  d_Y = BY(ggx,W,g) + BY(x,ggW,g)
//   d_x = Bx(ggY,W,g) + Bx(Y,ggW,g)                         (to senders)
// OUT: the outputs the kernel is built for (1 d_W, 2 d_Y, 4 d_grad_out, 8 d_x); a
// kernel for a subset holds fewer live registers.
// flags: bit0 d_W, bit1 d_Y, bit2 d_grad_out, bits 3-4 d_x mode (0 none, 1 atomic, 2 rows),
//        bits 5-8 add into d_W / d_Y / d_grad_out / the d_x rows instead of overwriting
// ---------------------------------------------------------------------------
constexpr int DW = 1, DY = 2, DGO = 4, DX = 8;

// Path groups: DS = false runs on the backward groups (BG, NGB), DS = true on the
// double-backward groups (DG, NGD), which the planner splits finer where the larger
// kernels need the registers. The fused kernels exist for both sets (oeq_dbwd_<t> and
// oeq_dbwd_<t>_d, the latter empty when the two sets are the same); the split passes run on
// DG. The host sizes each launch's grid by the kernel's set.
template <bool DS> struct DbwdSet { static constexpr int N = NGB; };
template <> struct DbwdSet<true> { static constexpr int N = NGD; };
template <bool DS, int G> struct DbwdGr { using T = BG<G>; };
template <int G> struct DbwdGr<true, G> { using T = DG<G>; };

template <int TM, int OUT, bool DS, int G>
__device__ __forceinline__ void dbwd_group(GyStage &st, int r, int wv, int u, const int *__restrict__ rowptr,
                                           const int *__restrict__ src, const real_t *__restrict__ x,
                                           const real_t *__restrict__ Y, const real_t *__restrict__ W,
                                           const real_t *__restrict__ g, const real_t *__restrict__ ggx,
                                           const real_t *__restrict__ ggY, const real_t *__restrict__ ggW,
                                           real_t *__restrict__ dx, real_t *__restrict__ dY,
                                           real_t *__restrict__ dW, real_t *__restrict__ dg, int flags) {
    using Gr = typename DbwdGr<DS, G>::T;
    const int lane = threadIdx.x & 63;
    const bool act = (U % 64 == 0) || (u < U);
    const int uu = act ? u : 0;
    const bool want_dw = (OUT & DW) && (flags & 1) != 0, want_dy = (OUT & DY) && (flags & 2) != 0,
               want_dg = (OUT & DGO) && (flags & 4) != 0;
    const int dxmode = (OUT & DX) ? (flags >> 3) & 3 : 0;
    // add into the outputs instead of overwriting (one pass per tangent)
    const bool acc_dw = (flags & 32) != 0, acc_dy = (flags & 64) != 0, acc_dg = (flags & 128) != 0,
               acc_h = (flags & 256) != 0;
    constexpr bool HAS_DX = (TM & 6) != 0 && (OUT & DX) != 0;
    constexpr bool GW_ = (OUT & DW) != 0, GY_ = (OUT & DY) != 0, GX_ = (OUT & DX) != 0;
    real_t gv[Gr::NO];
    Gr::load_g(g + (i64)r * OD, uu, gv);
    if (!act) zero(gv);
    real_t dgacc[Gr::NO];  // dropped by the compiler when OUT has no DGO
    zero(dgacc);
    const int e0 = uni(rowptr[r]), e1 = uni(rowptr[r + 1]);
    // per-edge operands (unused ones are dropped by the compiler for a given TM)
    struct Ops {
        real_t y[YD], x[Gr::NX], w[Gr::NW], tx[Gr::NX], ty[YD], tw[Gr::NW];
    };
    auto load = [&](int e, int s, Ops &o) {
        load_y(Y, e, o.y);
        Gr::load_x(x + (i64)s * XD, uu, o.x);
        Gr::load_w(W + (i64)e * (P * U), uu, o.w);
        if (TM & 1) Gr::load_x(ggx + (i64)s * XD, uu, o.tx);
        if (TM & 2) load_y(ggY, e, o.ty);
        if (TM & 4) Gr::load_w(ggW + (i64)e * (P * U), uu, o.tw);
    };
    if (e0 < e1) {
        int s = uni(src[e0]);
        Ops cur;
        load(e0, s, cur);
        for (int e = e0; e < e1; ++e) {
            const int en = (e + 1 < e1) ? e + 1 : e;
            const int sn = uni(src[en]);
            Ops nxt;
            load(en, sn, nxt);
            // keep the next edge's loads ahead of this edge's arithmetic
            PIN_BWD();
            const int j = uni((e - e0) % GY_TILE);
            real_t dw[Gr::NW], dy[YD], dxp[Gr::NX];
            zero(dw);
            zero(dy);
            zero(dxp);
            if constexpr (OUT == DW) {
                // the d_W-only pass, one tangent after the other: this order fits 256 registers
                // in fp64 (two waves per SIMD) where the interleaved one needs 258
                if constexpr ((TM & 1) != 0) Gr::template vjp<true, false, false>(cur.tx, cur.y, cur.w, gv, dw, dy, dxp);
                if constexpr ((TM & 2) != 0) Gr::template vjp<true, false, false>(cur.x, cur.ty, cur.w, gv, dw, dy, dxp);
            } else {
                // every term of this edge in one pass (the g contraction is shared by the tangents)
                Gr::template dbwd_edge<TM, GW_ && (TM & 3) != 0, GY_ && (TM & 5) != 0, GX_ && (TM & 6) != 0>(
                    cur.x, cur.y, cur.w, cur.tx, cur.ty, cur.tw, gv, (OUT & DGO) != 0 && want_dg, dgacc, dw, dy, dxp);
            }
            if (want_dw && act) {
                if (acc_dw)
                    Gr::add_w(dW + (i64)e * (P * U), u, dw);
                else
                    Gr::store_w(dW + (i64)e * (P * U), u, dw);
            }
            if (want_dy) {
                gy_push(st, dY, e, j, dy, lane, wv, acc_dy);
                if (j == GY_TILE - 1 || e + 1 == e1) gy_flush(st, dY, e - j, j + 1, acc_dy);
            }
            if (HAS_DX && dxmode == 1 && act) Gr::atomic_x(dx + (i64)s * GXD, u, dxp);
            if (HAS_DX && dxmode == 2 && act) {
                if (acc_h)
                    Gr::add_x(dx + (i64)e * GXD, u, dxp);
                else
                    Gr::store_x(dx + (i64)e * GXD, u, dxp);
            }
            s = sn;
            cur = nxt;
        }
    }
    if constexpr ((OUT & DGO) != 0) {
        if (want_dg && act) {
            if (acc_dg)
                Gr::add_out(dg + (i64)r * OD, u, dgacc);
            else
                Gr::store_out(dg + (i64)r * OD, u, dgacc);
        }
        // one-channel output blocks: the sum over the channels, as in the forward (each wave
        // adds its lanes, then the chunks of the receiver are added in LDS in chunk order);
        // want_dg is the same for every wave of the workgroup, so all meet at the barrier
        if constexpr (Gr::NSUM > 0) {
            if (want_dg) {
                __shared__ real_t red[UCH * (DBWD_NSUM_MAX > 0 ? DBWD_NSUM_MAX : 1)];
                real_t sv[Gr::NSUM];
                Gr::sum_pick(dgacc, sv);
#pragma unroll
                for (int j = 0; j < Gr::NSUM; ++j) {
                    const real_t t = wave_sum(act ? sv[j] : real_t(0));
                    if (lane == 0) red[wv * DBWD_NSUM_MAX + j] = t;
                }
                __syncthreads();
                for (int j = threadIdx.x; j < Gr::NSUM; j += blockDim.x) {
                    real_t t = red[j];
                    for (int c = 1; c < UCH; ++c) t += red[c * DBWD_NSUM_MAX + j];
                    real_t *q = dg + (i64)r * OD + Gr::sum_off_g(j);
                    *q = acc_dg ? *q + t : t;
                }
            }
        }
    }
}

template <int TM, int OUT, bool DS, int G>
__device__ __forceinline__ void dbwd_dispatch(GyStage &st, int r, int grp, int wv, int u, const int *__restrict__ rowptr,
                                              const int *__restrict__ src, const real_t *__restrict__ x,
                                              const real_t *__restrict__ Y, const real_t *__restrict__ W,
                                              const real_t *__restrict__ g, const real_t *__restrict__ ggx,
                                              const real_t *__restrict__ ggY, const real_t *__restrict__ ggW,
                                              real_t *__restrict__ dx, real_t *__restrict__ dY,
                                              real_t *__restrict__ dW, real_t *__restrict__ dg, int flags) {
    if (grp == G) {
        dbwd_group<TM, OUT, DS, G>(st, r, wv, u, rowptr, src, x, Y, W, g, ggx, ggY, ggW, dx, dY, dW, dg, flags);
        return;
    }
    if constexpr (G + 1 < DbwdSet<DS>::N)
        dbwd_dispatch<TM, OUT, DS, G + 1>(st, r, grp, wv, u, rowptr, src, x, Y, W, g, ggx, ggY, ggW, dx, dY, dW, dg,
                                      flags);
}

template <int TM, int OUT, bool DS>
__device__ __forceinline__ void dbwd_body(const int *__restrict__ rowptr, const int *__restrict__ src,
                                          const real_t *__restrict__ x, const real_t *__restrict__ Y,
                                          const real_t *__restrict__ W, const real_t *__restrict__ g,
                                          const real_t *__restrict__ ggx, const real_t *__restrict__ ggY,
                                          const real_t *__restrict__ ggW, real_t *__restrict__ dx,
                                          real_t *__restrict__ dY, real_t *__restrict__ dW,
                                          real_t *__restrict__ dg, int flags, i64 gy_stride, int n_nodes) {
    __shared__ GyStage st;
    constexpr int NG = DbwdSet<DS>::N;
    const int r = blockIdx.x / NG, grp = blockIdx.x - r * NG;
    if (r >= n_nodes) return;  // a grid larger than the kernel's groups x nodes reads nothing
    const int wv = uni(threadIdx.x >> 6);
    dbwd_dispatch<TM, OUT, DS, 0>(st, r, grp, wv, wv * 64 + (threadIdx.x & 63), rowptr, src, x, Y, W, g, ggx, ggY, ggW, dx,
                         dY + grp * gy_stride, dW, dg, flags);
}

// oeq_dbwd_<TM>: every output in one pass.  oeq_dbwd_<TM>_<OUT>: the passes of
// the split double backward (d_W; d_Y and d_x; d_grad_out is left to the
// forward kernel, one accumulating launch per tangent).
#define OEQ_DBWD_KERNEL(NAME, TM, OUT, DS)                                                          \
    extern "C" __global__ void __launch_bounds__(UCH * 64) BWD_OCCUPANCY NAME(                      \
        const int *__restrict__ rowptr, const int *__restrict__ src, const real_t *__restrict__ x, \
        const real_t *__restrict__ Y, const real_t *__restrict__ W, const real_t *__restrict__ g,  \
        const real_t *__restrict__ ggx, const real_t *__restrict__ ggY,                            \
        const real_t *__restrict__ ggW, real_t *__restrict__ dx, real_t *__restrict__ dY,          \
        real_t *__restrict__ dW, real_t *__restrict__ dg, int flags, i64 gy_stride, int n_nodes) { \
        if constexpr (!(DS && OUT == 15) || DBWD_TWO_SETS)                                         \
            dbwd_body<TM, OUT, DS>(rowptr, src, x, Y, W, g, ggx, ggY, ggW, dx, dY, dW, dg, flags,  \
                                   gy_stride, n_nodes);                                            \
    }
OEQ_DBWD_KERNEL(oeq_dbwd_1, 1, 15, false)
OEQ_DBWD_KERNEL(oeq_dbwd_2, 2, 15, false)
OEQ_DBWD_KERNEL(oeq_dbwd_3, 3, 15, false)
OEQ_DBWD_KERNEL(oeq_dbwd_4, 4, 15, false)
OEQ_DBWD_KERNEL(oeq_dbwd_5, 5, 15, false)
OEQ_DBWD_KERNEL(oeq_dbwd_6, 6, 15, false)
OEQ_DBWD_KERNEL(oeq_dbwd_7, 7, 15, false)
// the same on the double-backward groups (empty when they are the backward groups)
OEQ_DBWD_KERNEL(oeq_dbwd_1_d, 1, 15, true)
OEQ_DBWD_KERNEL(oeq_dbwd_2_d, 2, 15, true)
OEQ_DBWD_KERNEL(oeq_dbwd_3_d, 3, 15, true)
OEQ_DBWD_KERNEL(oeq_dbwd_4_d, 4, 15, true)
OEQ_DBWD_KERNEL(oeq_dbwd_5_d, 5, 15, true)
OEQ_DBWD_KERNEL(oeq_dbwd_6_d, 6, 15, true)
OEQ_DBWD_KERNEL(oeq_dbwd_7_d, 7, 15, true)
// d_W = BW(gg_x,Y,g) + BW(x,gg_Y,g): reads no weights
OEQ_DBWD_KERNEL(oeq_dbwd_1_1, 1, 1, true)
OEQ_DBWD_KERNEL(oeq_dbwd_2_1, 2, 1, true)
OEQ_DBWD_KERNEL(oeq_dbwd_3_1, 3, 1, true)
// d_Y and d_x of several tangents in one pass over W and gg_W
OEQ_DBWD_KERNEL(oeq_dbwd_3_10, 3, 10, true)
OEQ_DBWD_KERNEL(oeq_dbwd_5_10, 5, 10, true)
OEQ_DBWD_KERNEL(oeq_dbwd_6_10, 6, 10, true)
OEQ_DBWD_KERNEL(oeq_dbwd_7_10, 7, 10, true)
// one tangent: d_Y = BY(gg_x,W,g); d_x = Bx(gg_Y,W,g); d_Y, d_x = BY(x,gg_W,g), Bx(Y,gg_W,g)
OEQ_DBWD_KERNEL(oeq_dbwd_1_2, 1, 2, true)
OEQ_DBWD_KERNEL(oeq_dbwd_2_8, 2, 8, true)
OEQ_DBWD_KERNEL(oeq_dbwd_4_10, 4, 10, true)

// ---------------------------------------------------------------------------
// Hessian-vector product (tangent v = gg_x only) from Y-contracted CG rows.  The
// receiver's edges are taken in tiles of HVP_MT; for each tile the workgroup's lanes
// build the rows M[e] = C . Y[e] in LDS (one lane per edge), then every channel lane
// streams the tile: t = M^T v[s] per path gives d_grad_out += w t and d_W = g . t,
// and d_Y = w (v . C g) is formed from the tables and reduced like the VJP's Y
// gradient.  d_x is zero.  A workgroup is one (receiver, backward group), so all of
// its waves run the same tiles and meet at the same barriers.
// flags: bit0 d_W, bit1 d_Y, bit2 d_grad_out
// ---------------------------------------------------------------------------
template <int G>
__device__ __forceinline__ void hvp_group_lds(GyStage &st, real_t *__restrict__ mt, int r, int wv, int u,
                                              const int *__restrict__ rowptr, const int *__restrict__ src,
                                              const real_t *__restrict__ Y, const real_t *__restrict__ W,
                                              const real_t *__restrict__ g, const real_t *__restrict__ v,
                                              real_t *__restrict__ dY, real_t *__restrict__ dW,
                                              real_t *__restrict__ dg, int flags) {
    using Gr = BG<G>;
    const int lane = threadIdx.x & 63;
    const bool act = (U % 64 == 0) || (u < U);
    const int uu = act ? u : 0;
    const bool want_dw = (flags & 1) != 0, want_dy = (flags & 2) != 0, want_dg = (flags & 4) != 0;
    const int bi = wv * 64 + lane;  // the tile row this lane builds (when < HVP_MT)
    real_t gv[Gr::NO];
    Gr::load_g(g + (i64)r * OD, uu, gv);
    if (!act) zero(gv);
    real_t dgacc[Gr::NO];
    zero(dgacc);
    const int e0 = uni(rowptr[r]), e1 = uni(rowptr[r + 1]);
    if (e0 < e1) {
        int s = uni(src[e0]);
        real_t vv[Gr::NX], wv_[Gr::NW];
        Gr::load_x(v + (i64)s * XD, uu, vv);
        Gr::load_w(W + (i64)e0 * (P * U), uu, wv_);
        real_t ynone[YD];  // the Y values are in the M rows; dbwd_edge reads none for this tangent
        zero(ynone);
        int tb = e0;  // first edge of the tile whose rows are in LDS
        for (int e = e0; e < e1; ++e) {
            if (e == tb + HVP_MT || e == e0) {
                tb = e;
                __syncthreads();  // the previous tile's rows are no longer read
                if (bi < HVP_MT && e + bi < e1) {
                    real_t yv[YD];
                    load_y(Y, e + bi, yv);
                    Gr::make_m(yv, mt + bi * Gr::SM);
                }
                __syncthreads();
            }
            const int en = (e + 1 < e1) ? e + 1 : e;
            const int sn = uni(src[en]);
            real_t vn[Gr::NX], wn[Gr::NW];
            Gr::load_x(v + (i64)sn * XD, uu, vn);
            Gr::load_w(W + (i64)en * (P * U), uu, wn);
            PIN_BWD();
            const int j = uni((e - e0) % GY_TILE);
            real_t dw[Gr::NW], dy[YD], dxp[Gr::NX], tnone[Gr::NW];
            zero(dw);
            zero(dy);
            zero(dxp);
            zero(tnone);
            Gr::hvp_m(vv, mt + (e - tb) * Gr::SM, wv_, gv, dgacc, dw);
            if (want_dy)
                Gr::template dbwd_edge<1, false, true, false>(vv, ynone, wv_, vv, ynone, tnone, gv, false, dgacc, dw,
                                                              dy, dxp);
            if (want_dw && act) Gr::store_w(dW + (i64)e * (P * U), u, dw);
            if (want_dy) {
                gy_push(st, dY, e, j, dy, lane, wv);
                if (j == GY_TILE - 1 || e + 1 == e1) gy_flush(st, dY, e - j, j + 1);
            }
#pragma unroll
            for (int k = 0; k < Gr::NX; ++k) vv[k] = vn[k];
#pragma unroll
            for (int k = 0; k < Gr::NW; ++k) wv_[k] = wn[k];
        }
    }
    if (want_dg && act) Gr::store_out(dg + (i64)r * OD, u, dgacc);
}

template <int G>
__device__ __forceinline__ void hvp_dispatch(GyStage &st, real_t *__restrict__ mt, int r, int grp, int wv, int u,
                                             const int *__restrict__ rowptr, const int *__restrict__ src,
                                             const real_t *__restrict__ Y, const real_t *__restrict__ W,
                                             const real_t *__restrict__ g, const real_t *__restrict__ v,
                                             real_t *__restrict__ dY, real_t *__restrict__ dW,
                                             real_t *__restrict__ dg, int flags) {
    if constexpr (HVP_LDS) {
        if (grp == G) {
            hvp_group_lds<G>(st, mt, r, wv, u, rowptr, src, Y, W, g, v, dY, dW, dg, flags);
            return;
        }
        if constexpr (G + 1 < NGB) hvp_dispatch<G + 1>(st, mt, r, grp, wv, u, rowptr, src, Y, W, g, v, dY, dW, dg, flags);
    }
}

extern "C" __global__ void __launch_bounds__(UCH * 64) BWD_OCCUPANCY
oeq_hvp_lds(const int *__restrict__ rowptr, const int *__restrict__ src, const real_t *__restrict__ Y,
            const real_t *__restrict__ W, const real_t *__restrict__ g, const real_t *__restrict__ v,
            real_t *__restrict__ dY, real_t *__restrict__ dW, real_t *__restrict__ dg, int flags, i64 gy_stride,
            int n_nodes) {
    if constexpr (HVP_LDS) {
        __shared__ GyStage st;
        __shared__ __attribute__((aligned(16))) real_t mbuf[HVP_M_MAX * HVP_MT > 0 ? HVP_M_MAX * HVP_MT : 1];
        const int r = blockIdx.x / NGB, grp = blockIdx.x - r * NGB;
        if (r >= n_nodes) return;  // a grid larger than the groups x nodes reads nothing
        const int wv = uni(threadIdx.x >> 6);
        hvp_dispatch<0>(st, mbuf, r, grp, wv, wv * 64 + (threadIdx.x & 63), rowptr, src, Y, W, g, v,
                        dY + grp * gy_stride, dW, dg, flags);
    }
}
