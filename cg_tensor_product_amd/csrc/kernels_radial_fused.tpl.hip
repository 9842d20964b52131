// Forward and VJP that form the radial weights inside the convolution.

// ---------------------------------------------------------------------------
// Forward with the radial weights computed in the kernel (no W tensor): with a
// hidden layer of RH = 8 units, W[e, p, u] = sum_j h[e, j] W2[j, p, u] / sqrt(8).
// Each lane keeps its 8 x NW slice of W2 in registers (loaded once); per edge
// it reads the 8 hidden values (wave-uniform) and forms its W values, in place
// of streaming them.  h [E, 8] comes from oeq_radial_basis + oeq_radial_hidden.
// ---------------------------------------------------------------------------
constexpr int RH = 8;

template <int G>
__device__ __forceinline__ void fwd_radial_group(int r, int u, const int *__restrict__ rowptr,
                                                 const int *__restrict__ src, const real_t *__restrict__ x,
                                                 const real_t *__restrict__ Y, const real_t *__restrict__ hid,
                                                 const real_t *__restrict__ W2, real_t *__restrict__ out) {
    using Gr = FG<G>;
    const bool act = (U % 64 == 0) || (u < U);
    const int uu = act ? u : 0;
    real_t w2[RH][Gr::NW];
#pragma unroll
    for (int j = 0; j < RH; ++j) {
        Gr::load_wrow(W2 + (i64)j * (P * U), uu, w2[j]);
#pragma unroll
        for (int k = 0; k < Gr::NW; ++k) w2[j][k] *= real_t(0.35355339059327373);  // 1/sqrt(8)
    }
    real_t sum[Gr::NO];
    zero(sum);
    const int e0 = uni(rowptr[r]), e1 = uni(rowptr[r + 1]);
    if (e0 < e1) {
        int s = uni(src[e0]);
        real_t yv[YD], xv[Gr::NX], hv[RH];
        load_y(Y, e0, yv);
        Gr::load_x(x + (i64)s * XD, uu, xv);
#pragma unroll
        for (int j = 0; j < RH; ++j) hv[j] = hid[(i64)e0 * RH + j];
        for (int e = e0; e < e1; ++e) {
            real_t yn[YD], xn[Gr::NX], hn[RH];
            const int en = (e + 1 < e1) ? e + 1 : e;
            const int sn = uni(src[en]);
            load_y(Y, en, yn);
            Gr::load_x(x + (i64)sn * XD, uu, xn);
#pragma unroll
            for (int j = 0; j < RH; ++j) hn[j] = hid[(i64)en * RH + j];
            PIN_FWD();
            real_t wv[Gr::NW];
#pragma unroll
            for (int k = 0; k < Gr::NW; ++k) {
                real_t t = hv[0] * w2[0][k];
#pragma unroll
                for (int j = 1; j < RH; ++j) t = fmar(hv[j], w2[j][k], t);
                wv[k] = t;
            }
            Gr::edge(xv, yv, wv, sum);
#pragma unroll
            for (int q = 0; q < YD; ++q) yv[q] = yn[q];
#pragma unroll
            for (int q = 0; q < Gr::NX; ++q) xv[q] = xn[q];
#pragma unroll
            for (int q = 0; q < RH; ++q) hv[q] = hn[q];
        }
    }
    if (act) Gr::store_out(out + (i64)r * OD, u, sum);
}

template <int G>
__device__ __forceinline__ void fwd_radial_dispatch(int grp, int r, int u, const int *__restrict__ rowptr,
                                                    const int *__restrict__ src, const real_t *__restrict__ x,
                                                    const real_t *__restrict__ Y, const real_t *__restrict__ hid,
                                                    const real_t *__restrict__ W2, real_t *__restrict__ out) {
    if (grp == G) {
        fwd_radial_group<G>(r, u, rowptr, src, x, Y, hid, W2, out);
        return;
    }
    if constexpr (G + 1 < NGF) fwd_radial_dispatch<G + 1>(grp, r, u, rowptr, src, x, Y, hid, W2, out);
}

extern "C" __global__ void __launch_bounds__(UCH * NGF * 64) FWD_OCCUPANCY
oeq_fwd_radial(const int *__restrict__ rowptr, const int *__restrict__ src, const real_t *__restrict__ x,
               const real_t *__restrict__ Y, const real_t *__restrict__ hid, const real_t *__restrict__ W2,
               real_t *__restrict__ out, int n_nodes) {
    if ((int)blockIdx.x >= n_nodes) return;
    const int w = uni(threadIdx.x >> 6);
    const int grp = w / UCH, uc = w - grp * UCH;
    fwd_radial_dispatch<0>(grp, blockIdx.x, uc * 64 + (threadIdx.x & 63), rowptr, src, x, Y, hid, W2, out);
}

// VJP with the radial weights formed in the kernel (hidden width RH = 8).  Per
// edge, as oeq_bwd_* with W[e] = h[e] W2 / sqrt(8) formed from registers, and in
// place of grad_W:
//   dh[e, j]  = sum_{p,u} gW[e,p,u] W2[j,p,u] / sqrt(8)   (lanes, then waves, like gY)
//   dW2 partial of the workgroup: sum over its edges of h[e, j] gW[e,p,u] / sqrt(8),
//   stored as row r of dw2p[N, RH, P*U] and summed over receivers in order later.
// A workgroup is one (receiver, radial path group: RG<g>, NGR of them); with several
// groups the gY and dh rows are per-group partials, added in group order later.
// flags: bit0 dW2 partials, bit1 grad_Y, bit2 dh.  Needs PY >= RH (Y degrees >= 2).
template <int GXMODE, int G>
__device__ __forceinline__ void bwd_radial_group(GyStage &st, GyStage &sth, int r, int wv, int u,
                                                 const int *__restrict__ rowptr, const int *__restrict__ src,
                                                 const real_t *__restrict__ x, const real_t *__restrict__ Y,
                                                 const real_t *__restrict__ hid, const real_t *__restrict__ W2,
                                                 const real_t *__restrict__ g, real_t *__restrict__ gx,
                                                 real_t *__restrict__ gY, real_t *__restrict__ dh,
                                                 real_t *__restrict__ dw2p, int flags) {
    if constexpr (PY >= RH) {
        using Gr = RG<G>;
        const int lane = threadIdx.x & 63;
        const bool act = (U % 64 == 0) || (u < U);
        const int uu = act ? u : 0;
        const bool want_w2 = (flags & 1) != 0, want_gy = (flags & 2) != 0, want_dh = (flags & 4) != 0;
        real_t w2[RH][Gr::NW], dw2[RH][Gr::NW];
#pragma unroll
        for (int j = 0; j < RH; ++j) {
            Gr::load_wrow(W2 + (i64)j * (P * U), uu, w2[j]);
#pragma unroll
            for (int k = 0; k < Gr::NW; ++k) {
                w2[j][k] *= real_t(0.35355339059327373);  // 1/sqrt(8)
                dw2[j][k] = real_t(0);
            }
        }
        real_t gv[Gr::NO];
        Gr::load_g(g + (i64)r * OD, uu, gv);
        if (!act) zero(gv);  // inactive lanes contribute nothing to the lane sums
        const int e0 = uni(rowptr[r]), e1 = uni(rowptr[r + 1]);
        if (e0 < e1) {
            int s = uni(src[e0]);
            real_t yv[YD], xv[Gr::NX], hv[RH];
            load_y(Y, e0, yv);
            Gr::load_x(x + (i64)s * XD, uu, xv);
#pragma unroll
            for (int j = 0; j < RH; ++j) hv[j] = hid[(i64)e0 * RH + j];
            for (int e = e0; e < e1; ++e) {
                const int en = (e + 1 < e1) ? e + 1 : e;
                const int sn = uni(src[en]);
                real_t yn[YD], xn[Gr::NX], hn[RH];
                load_y(Y, en, yn);
                Gr::load_x(x + (i64)sn * XD, uu, xn);
#pragma unroll
                for (int j = 0; j < RH; ++j) hn[j] = hid[(i64)en * RH + j];
                PIN_BWD();
                const int jt = uni((e - e0) % GY_TILE);
                real_t wv_[Gr::NW];
#pragma unroll
                for (int k = 0; k < Gr::NW; ++k) {
                    real_t t = hv[0] * w2[0][k];
#pragma unroll
                    for (int j = 1; j < RH; ++j) t = fmar(hv[j], w2[j][k], t);
                    wv_[k] = t;
                }
                real_t gw[Gr::NW], gy[YD], gxp[Gr::NX];
                zero(gw);
                zero(gy);
                zero(gxp);
                Gr::template vjp<true, true, (GXMODE != 0)>(xv, yv, wv_, gv, gw, gy, gxp);
                if (!act) zero(gw);
                if (want_w2) {
#pragma unroll
                    for (int j = 0; j < RH; ++j)
#pragma unroll
                        for (int k = 0; k < Gr::NW; ++k) dw2[j][k] = fmar(hv[j], gw[k], dw2[j][k]);
                }
                if (want_dh) {
                    real_t d[RH];
#pragma unroll
                    for (int j = 0; j < RH; ++j) {
                        real_t t = real_t(0);
#pragma unroll
                        for (int k = 0; k < Gr::NW; ++k) t = fmar(gw[k], w2[j][k], t);
                        d[j] = t;
                    }
                    gy_push<RH>(sth, dh, e, jt, d, lane, wv);
                    if (jt == GY_TILE - 1 || e + 1 == e1) gy_flush<RH>(sth, dh, e - jt, jt + 1);
                }
                if (want_gy) {
                    gy_push(st, gY, e, jt, gy, lane, wv);
                    if (jt == GY_TILE - 1 || e + 1 == e1) gy_flush(st, gY, e - jt, jt + 1);
                }
                if (GXMODE == 1 && act) Gr::atomic_x(gx + (i64)s * GXD, u, gxp);
                if (GXMODE == 2 && act) Gr::store_x(gx + (i64)e * GXD, u, gxp);
                s = sn;
#pragma unroll
                for (int q = 0; q < YD; ++q) yv[q] = yn[q];
#pragma unroll
                for (int q = 0; q < Gr::NX; ++q) xv[q] = xn[q];
#pragma unroll
                for (int q = 0; q < RH; ++q) hv[q] = hn[q];
            }
        }
        if (want_w2 && act) {
#pragma unroll
            for (int j = 0; j < RH; ++j) {
#pragma unroll
                for (int k = 0; k < Gr::NW; ++k) dw2[j][k] *= real_t(0.35355339059327373);
                Gr::store_w(dw2p + ((i64)r * RH + j) * (P * U), u, dw2[j]);
            }
        }
    }
}

template <int GXMODE, int G>
__device__ __forceinline__ void bwd_radial_dispatch(GyStage &st, GyStage &sth, int r, int grp, int wv, int u,
                                                    const int *__restrict__ rowptr, const int *__restrict__ src,
                                                    const real_t *__restrict__ x, const real_t *__restrict__ Y,
                                                    const real_t *__restrict__ hid, const real_t *__restrict__ W2,
                                                    const real_t *__restrict__ g, real_t *__restrict__ gx,
                                                    real_t *__restrict__ gY, real_t *__restrict__ dh,
                                                    real_t *__restrict__ dw2p, int flags) {
    if (grp == G) {
        bwd_radial_group<GXMODE, G>(st, sth, r, wv, u, rowptr, src, x, Y, hid, W2, g, gx, gY, dh, dw2p, flags);
        return;
    }
    if constexpr (G + 1 < NGR)
        bwd_radial_dispatch<GXMODE, G + 1>(st, sth, r, grp, wv, u, rowptr, src, x, Y, hid, W2, g, gx, gY, dh, dw2p,
                                           flags);
}

#define OEQ_BWD_RADIAL_KERNEL(NAME, GXMODE)                                                              \
    extern "C" __global__ void __launch_bounds__(UCH * 64) BWD_OCCUPANCY NAME(                            \
        const int *__restrict__ rowptr, const int *__restrict__ src, const real_t *__restrict__ x,      \
        const real_t *__restrict__ Y, const real_t *__restrict__ hid, const real_t *__restrict__ W2,    \
        const real_t *__restrict__ g, real_t *__restrict__ gx, real_t *__restrict__ gY,                 \
        real_t *__restrict__ dh, real_t *__restrict__ dw2p, int flags, i64 gy_stride, i64 dh_stride,    \
        int n_nodes) {                                                                                  \
        __shared__ GyStage st, sth;                                                                     \
        const int r = blockIdx.x / NGR, grp = blockIdx.x - r * NGR;                                     \
        if (r >= n_nodes) return;                                                                       \
        const int wv = uni(threadIdx.x >> 6);                                                           \
        bwd_radial_dispatch<GXMODE, 0>(st, sth, r, grp, wv, wv * 64 + (threadIdx.x & 63), rowptr, src, x, Y, \
                                       hid, W2, g, gx, gY + grp * gy_stride, dh + grp * dh_stride, dw2p,  \
                                       flags);                                                          \
    }
OEQ_BWD_RADIAL_KERNEL(oeq_bwd_radial_nogx, 0)
OEQ_BWD_RADIAL_KERNEL(oeq_bwd_radial_atomic, 1)
OEQ_BWD_RADIAL_KERNEL(oeq_bwd_radial_rows, 2)
