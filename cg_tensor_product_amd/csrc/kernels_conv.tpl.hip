// Receiver-stationary passes: forward, VJP (three x-gradient modes), the
// ordered combination of partial rows and the per-sender sum of x-gradient rows.

// ---------------------------------------------------------------------------
// Forward: out[r] = sum over the receiver's edges of the per-edge messages.
// ---------------------------------------------------------------------------

// Output blocks of one channel receive the sum over the U channels.  Each wave adds its
// 64 lanes (inactive lanes give zero) and puts the total in LDS, slot [chunk][element];
// after every wave of the workgroup (all chunks of one receiver) has done so, the
// chunks are added in chunk order and the element is written.
__device__ __forceinline__ real_t *fwd_red() {
    __shared__ real_t red[NSUMT > 0 ? UCH * NSUMT : 1];
    return red;
}

template <class Gr>
__device__ __forceinline__ void fwd_sum_partial(const real_t (&sum)[Gr::NO], bool act, int uc, int lane) {
    real_t s[Gr::NSUM > 0 ? Gr::NSUM : 1];
    Gr::sum_pick(sum, s);
    real_t *red = fwd_red();
#pragma unroll
    for (int j = 0; j < Gr::NSUM; ++j) {
        const real_t t = wave_sum(act ? s[j] : real_t(0));
        if (lane == 0) red[uc * NSUMT + Gr::SOFF + j] = t;
    }
}

static_assert(NSUMT == 0 || !FWD_XCD, "the channel sum needs every chunk of a receiver in one workgroup");

// Every wave of the workgroup calls this once, after its group's partials.
__device__ __forceinline__ void fwd_sum_finish(int r, real_t *__restrict__ out, bool acc) {
    if constexpr (NSUMT > 0) {
        __syncthreads();
        const real_t *red = fwd_red();
        for (int t = threadIdx.x; t < NSUMT; t += blockDim.x) {
            real_t s = red[t];
            for (int c = 1; c < UCH; ++c) s += red[c * NSUMT + t];
            real_t *q = out + (i64)r * OD + sum_off(t);
            *q = acc ? *q + s : s;
        }
    }
}

template <int G, int YM>
__device__ __forceinline__ void fwd_group(int r, int u, const int *__restrict__ rowptr,
                                          const int *__restrict__ src, const real_t *__restrict__ x,
                                          const real_t *__restrict__ Y, const real_t *__restrict__ W,
                                          real_t *__restrict__ out, bool acc) {
    using Gr = FG<G>;
    const bool act = (U % 64 == 0) || (u < U);
    const int uu = act ? u : 0;  // inactive lanes read channel 0 and store nothing
    real_t sum[Gr::NO];
    zero(sum);
    const int e0 = uni(rowptr[r]), e1 = uni(rowptr[r + 1]);
    if (e0 < e1) {
        real_t pr[3] = {real_t(0), real_t(0), real_t(0)};  // the receiver's position (YM_POS)
        if constexpr (YM == YM_POS) {
#pragma unroll
            for (int c = 0; c < 3; ++c) pr[c] = Y[(i64)r * 3 + c];
        }
        // software pipeline: the next edge's loads are in flight while this one computes
        int s = uni(src[e0]);
        real_t yv[YD], xv[Gr::NX], wv[Gr::NW];
        edge_y<YM>(Y, e0, s, pr, yv);
        Gr::load_x(x + (i64)s * XD, uu, xv);
        Gr::load_w(W + (i64)e0 * (P * U), uu, wv);
        if constexpr (FWD_PF >= 2) {
            // two edges ahead: the loads of edges e+1 and e+2 are in flight while e computes
            // (the last edges reload the row's last edge rather than read past the row)
            const int ea = (e0 + 1 < e1) ? e0 + 1 : e0;
            const int sa = uni(src[ea]);
            real_t ya[YD], xa[Gr::NX], wa[Gr::NW];
            edge_y<YM>(Y, ea, sa, pr, ya);
            Gr::load_x(x + (i64)sa * XD, uu, xa);
            Gr::load_w(W + (i64)ea * (P * U), uu, wa);
            for (int e = e0; e < e1; ++e) {
                real_t yn[YD], xn[Gr::NX], wn[Gr::NW];
                const int en = (e + 2 < e1) ? e + 2 : e1 - 1;
                const int sn = uni(src[en]);
                edge_y<YM>(Y, en, sn, pr, yn);
                Gr::load_x(x + (i64)sn * XD, uu, xn);
                Gr::load_w(W + (i64)en * (P * U), uu, wn);
                PIN_FWD();
                Gr::edge(xv, yv, wv, sum);
#pragma unroll
                for (int k = 0; k < YD; ++k) { yv[k] = ya[k]; ya[k] = yn[k]; }
#pragma unroll
                for (int k = 0; k < Gr::NX; ++k) { xv[k] = xa[k]; xa[k] = xn[k]; }
#pragma unroll
                for (int k = 0; k < Gr::NW; ++k) { wv[k] = wa[k]; wa[k] = wn[k]; }
            }
        } else
        for (int e = e0; e < e1; ++e) {
            real_t yn[YD], xn[Gr::NX], wn[Gr::NW];
            const int en = (e + 1 < e1) ? e + 1 : e;
            const int sn = uni(src[en]);
            edge_y<YM>(Y, en, sn, pr, yn);
            Gr::load_x(x + (i64)sn * XD, uu, xn);
            Gr::load_w(W + (i64)en * (P * U), uu, wn);
            // keep the next edge's loads ahead of this edge's arithmetic
            PIN_FWD();
            Gr::edge(xv, yv, wv, sum);
#pragma unroll
            for (int k = 0; k < YD; ++k) yv[k] = yn[k];
#pragma unroll
            for (int k = 0; k < Gr::NX; ++k) xv[k] = xn[k];
#pragma unroll
            for (int k = 0; k < Gr::NW; ++k) wv[k] = wn[k];
        }
    }
    if (act) {
        if (acc)
            Gr::add_out(out + (i64)r * OD, u, sum);
        else
            Gr::store_out(out + (i64)r * OD, u, sum);
    }
    if constexpr (Gr::NSUM > 0) fwd_sum_partial<Gr>(sum, act, u >> 6, u & 63);
}

template <int G, int YM>
__device__ __forceinline__ void fwd_dispatch(int grp, int r, int u, const int *__restrict__ rowptr,
                                             const int *__restrict__ src, const real_t *__restrict__ x,
                                             const real_t *__restrict__ Y, const real_t *__restrict__ W,
                                             real_t *__restrict__ out, bool acc) {
    if (grp == G) {
        fwd_group<G, YM>(r, u, rowptr, src, x, Y, W, out, acc);
        return;
    }
    if constexpr (G + 1 < NGF) fwd_dispatch<G + 1, YM>(grp, r, u, rowptr, src, x, Y, W, out, acc);
}

// Forward from Y-contracted CG rows: the receiver's edges are taken in tiles of FWD_MT.
// For each tile the first waves of every group build the group's rows M[e] = C . Y[e] in
// LDS (one lane per edge), and every channel lane streams the tile's edges reading M[e] by
// broadcast.  Every wave of the workgroup has the same receiver, so all run the same tiles
// and meet at the same barriers.
template <int G>
__device__ __forceinline__ void fwd_group_lds(real_t *__restrict__ mt, int r, int uc, int lane, int bi,
                                              const int *__restrict__ rowptr, const int *__restrict__ src,
                                              const real_t *__restrict__ x, const real_t *__restrict__ Y,
                                              const real_t *__restrict__ W, real_t *__restrict__ out, bool acc) {
    using Gr = FG<G>;
    const int u = uc * 64 + lane;
    const bool act = (U % 64 == 0) || (u < U);
    const int uu = act ? u : 0;  // inactive lanes read channel 0 and store nothing
    const int i = bi;            // the tile row this lane builds (when < FWD_MT)
    real_t sum[Gr::NO];
    zero(sum);
    const int e0 = uni(rowptr[r]), e1 = uni(rowptr[r + 1]);
    if (e0 < e1) {
        int s = uni(src[e0]);
        real_t xv[Gr::NX], wv[Gr::NW];
        Gr::load_x(x + (i64)s * XD, uu, xv);
        Gr::load_w(W + (i64)e0 * (P * U), uu, wv);
        int tb = e0;  // first edge of the tile whose rows are in LDS
        for (int e = e0; e < e1; ++e) {
            if (e == tb + FWD_MT || e == e0) {
                tb = e;
                __syncthreads();  // the previous tile's rows are no longer read
                if (i < FWD_MT && e + i < e1) {
                    real_t yv[YD];
                    const real_t *yr = Y + (i64)(e + i) * YD;
#pragma unroll
                    for (int k = 0; k < YD; ++k) yv[k] = yr[k];
                    Gr::make_m(yv, mt + i * Gr::SM);
                }
                __syncthreads();
            }
            real_t xn[Gr::NX], wn[Gr::NW];
            const int en = (e + 1 < e1) ? e + 1 : e;
            const int sn = uni(src[en]);
            Gr::load_x(x + (i64)sn * XD, uu, xn);
            Gr::load_w(W + (i64)en * (P * U), uu, wn);
            PIN_FWD();
            Gr::edge_m(xv, mt + (e - tb) * Gr::SM, wv, sum);
#pragma unroll
            for (int k = 0; k < Gr::NX; ++k) xv[k] = xn[k];
#pragma unroll
            for (int k = 0; k < Gr::NW; ++k) wv[k] = wn[k];
        }
    }
    if (act) {
        if (acc)
            Gr::add_out(out + (i64)r * OD, u, sum);
        else
            Gr::store_out(out + (i64)r * OD, u, sum);
    }
    if constexpr (Gr::NSUM > 0) fwd_sum_partial<Gr>(sum, act, uc, lane);
}

template <int G>
__device__ __forceinline__ void fwd_lds_dispatch(real_t *__restrict__ mbuf, int grp, int r, int uc, int lane, int bi,
                                                 const int *__restrict__ rowptr, const int *__restrict__ src,
                                                 const real_t *__restrict__ x, const real_t *__restrict__ Y,
                                                 const real_t *__restrict__ W, real_t *__restrict__ out, bool acc) {
    if constexpr (FWD_LDS) {
        if (grp == G) {
            fwd_group_lds<G>(mbuf + FG<G>::MOFF * FWD_MT, r, uc, lane, bi, rowptr, src, x, Y, W, out, acc);
            return;
        }
        if constexpr (G + 1 < NGF) fwd_lds_dispatch<G + 1>(mbuf, grp, r, uc, lane, bi, rowptr, src, x, Y, W, out, acc);
    }
}

// Workgroup shape of oeq_fwd: all 64-channel chunks of a receiver (waves = chunks x path
// groups), or with FWD_XCD one chunk per workgroup (waves = path groups).
constexpr int FWD_WG = (FWD_XCD ? 1 : UCH) * NGF * 64;

extern "C" __global__ void __launch_bounds__(FWD_WG) FWD_OCCUPANCY
oeq_fwd(const int *__restrict__ rowptr, const int *__restrict__ src, const real_t *__restrict__ x,
        const real_t *__restrict__ Y, const real_t *__restrict__ W, real_t *__restrict__ out, int flags,
        int n_nodes) {
    // flags: bit0 add into out instead of overwriting it
    const int w = uni(threadIdx.x >> 6), lane = threadIdx.x & 63;
    int r, grp, uc, wc;  // receiver, path group, channel chunk, chunk index inside the workgroup
    if constexpr (FWD_XCD) {
        // Workgroup b is dispatched to XCD b % 8.  With UCH dividing 8, chunk c runs only on
        // the 8 / UCH XCDs with b % 8 % UCH == c, so each XCD's L2 holds the x rows of one
        // chunk (x[:, chunk] rather than all of x).
        const int b = blockIdx.x;
        if constexpr (8 % UCH == 0) {
            const int xcd = b & 7;
            uc = xcd % UCH;
            r = (b >> 3) * (8 / UCH) + xcd / UCH;
        } else {
            uc = b % UCH;
            r = b / UCH;
        }
        if (r >= n_nodes) return;
        grp = w;
        wc = 0;
    } else {
        grp = w / UCH;
        uc = w - grp * UCH;
        r = blockIdx.x;
        if (r >= n_nodes) return;
        wc = uc;
    }
    if constexpr (FWD_LDS) {
        __shared__ __attribute__((aligned(16))) real_t mbuf[FWD_M_ELEMS * FWD_MT > 0 ? FWD_M_ELEMS * FWD_MT : 1];
        fwd_lds_dispatch<0>(mbuf, grp, r, uc, lane, wc * 64 + lane, rowptr, src, x, Y, W, out, (flags & 1) != 0);
    } else {
        fwd_dispatch<0, YM_TENSOR>(grp, r, uc * 64 + lane, rowptr, src, x, Y, W, out, (flags & 1) != 0);
    }
    fwd_sum_finish(r, out, (flags & 1) != 0);
}

// The forward with Y evaluated in the kernel from the edge vectors vec[E, 3]
// (no Y tensor): each wave computes the harmonics of the edge it streams.
extern "C" __global__ void __launch_bounds__(UCH * NGF * 64) FWD_OCCUPANCY
oeq_fwd_vec(const int *__restrict__ rowptr, const int *__restrict__ src, const real_t *__restrict__ x,
            const real_t *__restrict__ vec, const real_t *__restrict__ W, real_t *__restrict__ out, int n_nodes) {
    if ((int)blockIdx.x >= n_nodes) return;
    const int w = uni(threadIdx.x >> 6);
    const int grp = w / UCH, uc = w - grp * UCH;
    fwd_dispatch<0, YM_VEC>(grp, blockIdx.x, uc * 64 + (threadIdx.x & 63), rowptr, src, x, vec, W, out, false);
    fwd_sum_finish(blockIdx.x, out, false);
}

// The forward from atom positions pos[N, 3]: the harmonics of edge e are those of
// pos[src[e]] - pos[r], evaluated in the kernel (no vector or Y tensor).
extern "C" __global__ void __launch_bounds__(UCH * NGF * 64) FWD_OCCUPANCY
oeq_fwd_pos(const int *__restrict__ rowptr, const int *__restrict__ src, const real_t *__restrict__ x,
            const real_t *__restrict__ pos, const real_t *__restrict__ W, real_t *__restrict__ out, int n_nodes) {
    if ((int)blockIdx.x >= n_nodes) return;
    const int w = uni(threadIdx.x >> 6);
    const int grp = w / UCH, uc = w - grp * UCH;
    fwd_dispatch<0, YM_POS>(grp, blockIdx.x, uc * 64 + (threadIdx.x & 63), rowptr, src, x, pos, W, out, false);
    fwd_sum_finish(blockIdx.x, out, false);
}

// The atomic x-gradient is accumulated m-major inside each x block (so the
// lanes of one atomic instruction address consecutive words); this restores the
// u-major row layout in place, one node row per workgroup.
extern "C" __global__ void __launch_bounds__(256)
oeq_x_untranspose(real_t *__restrict__ gx) {
    __shared__ real_t t[XT ? GXD : 1];
    real_t *row = gx + (i64)blockIdx.x * GXD;
    if (!XT) return;
    for (int i = threadIdx.x; i < GXD; i += 256) t[i] = row[i];
    __syncthreads();
    g_untranspose_row(t, row);
}

// ---------------------------------------------------------------------------
// Y-gradient staging: per-wave lane-reduced rows in LDS, summed over the waves
// of the workgroup (fixed order) every GY_TILE edges.  In the backward passes a
// workgroup is one (receiver, path group); with several groups each writes its
// partial Y-gradient rows to its own slice of the workspace and oeq_gy_combine
// adds the slices in group order.
// ---------------------------------------------------------------------------
struct GyStage {
    real_t red[UCH][GY_TILE][PY];
};

// Rows of width RW <= PY (default: the Y width); the radial VJP also stages its
// 8-wide hidden-value gradients this way.
template <int RW = YD>
__device__ __forceinline__ void gy_push(GyStage &st, real_t *__restrict__ gY, int e, int j,
                                        real_t (&gy)[RW], int lane, int wv, bool acc = false) {
    static_assert(RW <= PY, "row wider than the reduction");
    real_t v[PY];
#pragma unroll
    for (int k = 0; k < PY; ++k) v[k] = (k < RW) ? gy[k] : real_t(0);
    wave_reduce_scatter(v, lane);
    const int idx = lane >> (6 - LGPY);
    const bool writer = (lane & ((1 << (6 - LGPY)) - 1)) == 0;
    if (UCH == 1) {
        if (writer && idx < RW) gY[(i64)e * RW + idx] = acc ? gY[(i64)e * RW + idx] + v[0] : v[0];
    } else {
        if (writer) st.red[wv][j][idx] = v[0];
    }
}

template <int RW = YD>
__device__ __forceinline__ void gy_flush(GyStage &st, real_t *__restrict__ gY, int base, int n, bool acc = false) {
    if (UCH == 1) return;
    __syncthreads();
    for (int k = threadIdx.x; k < n * RW; k += UCH * 64) {
        const int j = k / RW, m = k - j * RW;
        real_t s = st.red[0][j][m];
#pragma unroll
        for (int w = 1; w < UCH; ++w) s += st.red[w][j][m];
        real_t *dst = gY + (i64)(base + j) * RW + m;
        *dst = acc ? *dst + s : s;
    }
    __syncthreads();
}

// flags: bit0 store grad_W, bit1 store grad_Y
// GXMODE: 0 no x gradient, 1 atomic add into gx[src[e]], 2 store row h[e] (summed per sender later)
template <int GXMODE, int G>
__device__ __forceinline__ void bwd_group(GyStage &st, int r, int wv, int u, const int *__restrict__ rowptr,
                                          const int *__restrict__ src, const real_t *__restrict__ x,
                                          const real_t *__restrict__ Y, const real_t *__restrict__ W,
                                          const real_t *__restrict__ g, real_t *__restrict__ gx,
                                          real_t *__restrict__ gY, real_t *__restrict__ gW, int flags) {
    using Gr = BG<G>;
    const int lane = threadIdx.x & 63;
    const bool act = (U % 64 == 0) || (u < U);
    const int uu = act ? u : 0;
    const bool want_gw = (flags & 1) != 0, want_gy = (flags & 2) != 0;
    real_t gv[Gr::NO];
    Gr::load_g(g + (i64)r * OD, uu, gv);
    if (!act) zero(gv);  // inactive lanes contribute nothing to the lane sums
    const int e0 = uni(rowptr[r]), e1 = uni(rowptr[r + 1]);
    if (e0 >= e1) return;
    // one edge's gradients from its loaded operands
    auto body = [&](int e, int s_, const real_t (&y_)[YD], const real_t (&x_)[Gr::NX], const real_t (&w_)[Gr::NW]) {
        const int j = uni((e - e0) % GY_TILE);
        real_t gw[Gr::NW], gy[YD], gxp[Gr::NX];
        zero(gw);
        zero(gy);
        zero(gxp);
        Gr::template vjp<true, true, (GXMODE != 0)>(x_, y_, w_, gv, gw, gy, gxp);
        if (want_gw && act) Gr::store_w(gW + (i64)e * (P * U), u, gw);
        if (want_gy) {
            gy_push(st, gY, e, j, gy, lane, wv);
            if (j == GY_TILE - 1 || e + 1 == e1) gy_flush(st, gY, e - j, j + 1);
        }
        if (GXMODE == 1 && act) Gr::atomic_x(gx + (i64)s_ * GXD, u, gxp);
        if (GXMODE == 2 && act) Gr::store_x(gx + (i64)e * GXD, u, gxp);
    };
    // software pipeline: the next edge's loads (BWD_PF = 2: the next two edges') are in
    // flight while this one computes
    int s = uni(src[e0]);
    real_t yv[YD], xv[Gr::NX], wv_[Gr::NW];
    load_y(Y, e0, yv);
    Gr::load_x(x + (i64)s * XD, uu, xv);
    Gr::load_w(W + (i64)e0 * (P * U), uu, wv_);
    if constexpr (BWD_PF >= 2) {
        // the last edges reload the row's last edge rather than read past the row
        const int ea = (e0 + 1 < e1) ? e0 + 1 : e0;
        int sa = uni(src[ea]);
        real_t ya[YD], xa[Gr::NX], wa[Gr::NW];
        load_y(Y, ea, ya);
        Gr::load_x(x + (i64)sa * XD, uu, xa);
        Gr::load_w(W + (i64)ea * (P * U), uu, wa);
        for (int e = e0; e < e1; ++e) {
            const int en = (e + 2 < e1) ? e + 2 : e1 - 1;
            const int sn = uni(src[en]);
            real_t yn[YD], xn[Gr::NX], wn[Gr::NW];
            load_y(Y, en, yn);
            Gr::load_x(x + (i64)sn * XD, uu, xn);
            Gr::load_w(W + (i64)en * (P * U), uu, wn);
            PIN_BWD();
            body(e, s, yv, xv, wv_);
            s = sa;
            sa = sn;
#pragma unroll
            for (int k = 0; k < YD; ++k) { yv[k] = ya[k]; ya[k] = yn[k]; }
#pragma unroll
            for (int k = 0; k < Gr::NX; ++k) { xv[k] = xa[k]; xa[k] = xn[k]; }
#pragma unroll
            for (int k = 0; k < Gr::NW; ++k) { wv_[k] = wa[k]; wa[k] = wn[k]; }
        }
    } else {
        for (int e = e0; e < e1; ++e) {
            const int en = (e + 1 < e1) ? e + 1 : e;
            const int sn = uni(src[en]);
            real_t yn[YD], xn[Gr::NX], wn[Gr::NW];
            load_y(Y, en, yn);
            Gr::load_x(x + (i64)sn * XD, uu, xn);
            Gr::load_w(W + (i64)en * (P * U), uu, wn);
            // keep the next edge's loads ahead of this edge's arithmetic
            PIN_BWD();
            body(e, s, yv, xv, wv_);
            s = sn;
#pragma unroll
            for (int k = 0; k < YD; ++k) yv[k] = yn[k];
#pragma unroll
            for (int k = 0; k < Gr::NX; ++k) xv[k] = xn[k];
#pragma unroll
            for (int k = 0; k < Gr::NW; ++k) wv_[k] = wn[k];
        }
    }
}

template <int GXMODE, int G>
__device__ __forceinline__ void bwd_dispatch(GyStage &st, int r, int grp, int wv, int u, const int *__restrict__ rowptr,
                                             const int *__restrict__ src, const real_t *__restrict__ x,
                                             const real_t *__restrict__ Y, const real_t *__restrict__ W,
                                             const real_t *__restrict__ g, real_t *__restrict__ gx,
                                             real_t *__restrict__ gY, real_t *__restrict__ gW, int flags) {
    if (grp == G) {
        bwd_group<GXMODE, G>(st, r, wv, u, rowptr, src, x, Y, W, g, gx, gY, gW, flags);
        return;
    }
    if constexpr (G + 1 < NGB)
        bwd_dispatch<GXMODE, G + 1>(st, r, grp, wv, u, rowptr, src, x, Y, W, g, gx, gY, gW, flags);
}

template <int GXMODE>
__device__ __forceinline__ void bwd_body(const int *__restrict__ rowptr, const int *__restrict__ src,
                                         const real_t *__restrict__ x, const real_t *__restrict__ Y,
                                         const real_t *__restrict__ W, const real_t *__restrict__ g,
                                         real_t *__restrict__ gx, real_t *__restrict__ gY,
                                         real_t *__restrict__ gW, int flags, i64 gy_stride, int n_nodes) {
    __shared__ GyStage st;
    const int r = blockIdx.x / NGB, grp = blockIdx.x - r * NGB;
    if (r >= n_nodes) return;  // a grid larger than the plan's groups x nodes reads nothing
    const int wv = uni(threadIdx.x >> 6);
    bwd_dispatch<GXMODE, 0>(st, r, grp, wv, wv * 64 + (threadIdx.x & 63), rowptr, src, x, Y, W, g, gx,
                            gY + grp * gy_stride, gW, flags);
}

extern "C" __global__ void __launch_bounds__(UCH * 64) BWD_OCCUPANCY
oeq_bwd_nogx(const int *__restrict__ rowptr, const int *__restrict__ src, const real_t *__restrict__ x,
             const real_t *__restrict__ Y, const real_t *__restrict__ W, const real_t *__restrict__ g,
             real_t *__restrict__ gx, real_t *__restrict__ gY, real_t *__restrict__ gW, int flags, i64 gy_stride,
             int n_nodes) {
    bwd_body<0>(rowptr, src, x, Y, W, g, gx, gY, gW, flags, gy_stride, n_nodes);
}

extern "C" __global__ void __launch_bounds__(UCH * 64) BWD_OCCUPANCY
oeq_bwd_atomic(const int *__restrict__ rowptr, const int *__restrict__ src, const real_t *__restrict__ x,
               const real_t *__restrict__ Y, const real_t *__restrict__ W, const real_t *__restrict__ g,
               real_t *__restrict__ gx, real_t *__restrict__ gY, real_t *__restrict__ gW, int flags, i64 gy_stride,
               int n_nodes) {
    bwd_body<1>(rowptr, src, x, Y, W, g, gx, gY, gW, flags, gy_stride, n_nodes);
}

extern "C" __global__ void __launch_bounds__(UCH * 64) BWD_OCCUPANCY
oeq_bwd_rows(const int *__restrict__ rowptr, const int *__restrict__ src, const real_t *__restrict__ x,
             const real_t *__restrict__ Y, const real_t *__restrict__ W, const real_t *__restrict__ g,
             real_t *__restrict__ h, real_t *__restrict__ gY, real_t *__restrict__ gW, int flags, i64 gy_stride,
             int n_nodes) {
    bwd_body<2>(rowptr, src, x, Y, W, g, h, gY, gW, flags, gy_stride, n_nodes);
}

// Partial rows of several groups added in group order: out[i] = sum_g part[g n + i].
extern "C" __global__ void __launch_bounds__(256)
oeq_part_combine(const real_t *__restrict__ part, int groups, real_t *__restrict__ out, i64 n) {
    for (i64 i = (i64)blockIdx.x * blockDim.x + threadIdx.x; i < n; i += (i64)gridDim.x * blockDim.x) {
        real_t s = part[i];
        for (int gidx = 1; gidx < groups; ++gidx) s += part[gidx * n + i];
        out[i] = s;
    }
}

// Y-gradient of several path groups: gY = sum over groups of the partial rows,
// in group order.
extern "C" __global__ void __launch_bounds__(256)
oeq_gy_combine(const real_t *__restrict__ part, real_t *__restrict__ gY, i64 n) {
    for (i64 i = (i64)blockIdx.x * blockDim.x + threadIdx.x; i < n; i += (i64)gridDim.x * blockDim.x) {
        real_t s = part[i];
#pragma unroll
        for (int gidx = 1; gidx < NGB; ++gidx) s += part[gidx * n + i];
        gY[i] = s;
    }
}

// ---------------------------------------------------------------------------
// Deterministic x gradient: gx[s] = sum of h[e] over the sender's edges, in the
// sender CSR's (increasing edge id) order.  Rows of GXD values (U channels in every
// block); with one-channel x blocks the caller passes rows in the workspace and
// oeq_fold_x then sums their channels.
// ---------------------------------------------------------------------------
extern "C" __global__ void __launch_bounds__(256)
oeq_sender_sum(const int *__restrict__ srowptr, const int *__restrict__ sperm,
               const real_t *__restrict__ h, real_t *__restrict__ gx, int n_nodes) {
    const int s = blockIdx.x;
    if (s >= n_nodes) return;
    const int k0 = uni(srowptr[s]), k1 = uni(srowptr[s + 1]);
    for (i64 c = threadIdx.x; c < GXD; c += 256) {
        real_t acc = real_t(0);
        int k = k0;
        // eight rows in flight, added in edge order
        for (; k + 8 <= k1; k += 8) {
            real_t t[8];
#pragma unroll
            for (int j = 0; j < 8; ++j) t[j] = h[(i64)uni(sperm[k + j]) * GXD + c];
#pragma unroll
            for (int j = 0; j < 8; ++j) acc += t[j];
        }
        for (; k < k1; ++k) acc += h[(i64)uni(sperm[k]) * GXD + c];
        gx[(i64)s * GXD + c] = acc;
    }
}

// x gradient of the atomic passes: rows with U channels in every block (gxe) to the
// x layout, a one-channel block taking the sum of its channels.
extern "C" __global__ void __launch_bounds__(256)
oeq_fold_x(const real_t *__restrict__ gxe, real_t *__restrict__ gx, i64 n) {
    for (i64 i = (i64)blockIdx.x * blockDim.x + threadIdx.x; i < n; i += (i64)gridDim.x * blockDim.x) {
        const i64 r = i / XD;
        gx[i] = fold_x_elem(gxe + r * GXD, (int)(i - r * XD));
    }
}
