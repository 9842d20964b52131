// Sender-stationary passes.

// ---------------------------------------------------------------------------
// Sender-stationary schedule.  The edges are visited through the sender view of
// the graph: srowptr/sperm (edge ids grouped by sender, increasing) and sdst (the
// receiver of each of those edges).  A workgroup owns one sender and keeps its x
// row in registers.
//   forward: each out-edge's message is added into out[receiver] with atomics,
//            m-major inside each output block (oeq_out_untranspose reorders);
//   VJP:     g[receiver] is gathered per edge; gW and gY are per edge as in the
//            receiver-stationary pass; gx of the sender is accumulated in registers
//            and stored once (no atomics, no workspace).
// ---------------------------------------------------------------------------
template <int G>
__device__ __forceinline__ void fwd_sender_group(int s, int u, const int *__restrict__ srowptr,
                                                 const int *__restrict__ sperm, const int *__restrict__ sdst,
                                                 const real_t *__restrict__ x, const real_t *__restrict__ Y,
                                                 const real_t *__restrict__ W, real_t *__restrict__ out) {
    using Gr = FG<G>;
    const bool act = (U % 64 == 0) || (u < U);
    const int uu = act ? u : 0;
    const int k0 = uni(srowptr[s]), k1 = uni(srowptr[s + 1]);
    if (k0 >= k1) return;
    real_t xv[Gr::NX];
    Gr::load_x(x + (i64)s * XD, uu, xv);
    int e = uni(sperm[k0]), r = uni(sdst[k0]);
    real_t yv[YD], wv[Gr::NW];
    load_y(Y, e, yv);
    Gr::load_w(W + (i64)e * (P * U), uu, wv);
    for (int k = k0; k < k1; ++k) {
        const int kn = (k + 1 < k1) ? k + 1 : k;
        const int en = uni(sperm[kn]), rn = uni(sdst[kn]);
        real_t yn[YD], wn[Gr::NW];
        load_y(Y, en, yn);
        Gr::load_w(W + (i64)en * (P * U), uu, wn);
        PIN_FWD();
        real_t msg[Gr::NO];
        zero(msg);
        Gr::edge(xv, yv, wv, msg);
        if (act) Gr::atomic_out(out + (i64)r * OD, u, msg);
        e = en;
        r = rn;
#pragma unroll
        for (int q = 0; q < YD; ++q) yv[q] = yn[q];
#pragma unroll
        for (int q = 0; q < Gr::NW; ++q) wv[q] = wn[q];
    }
}

template <int G>
__device__ __forceinline__ void fwd_sender_dispatch(int grp, int s, int u, const int *__restrict__ srowptr,
                                                    const int *__restrict__ sperm, const int *__restrict__ sdst,
                                                    const real_t *__restrict__ x, const real_t *__restrict__ Y,
                                                    const real_t *__restrict__ W, real_t *__restrict__ out) {
    if (grp == G) {
        fwd_sender_group<G>(s, u, srowptr, sperm, sdst, x, Y, W, out);
        return;
    }
    if constexpr (G + 1 < NGF) fwd_sender_dispatch<G + 1>(grp, s, u, srowptr, sperm, sdst, x, Y, W, out);
}

extern "C" __global__ void __launch_bounds__(UCH * NGF * 64) FWD_OCCUPANCY
oeq_fwd_sender(const int *__restrict__ srowptr, const int *__restrict__ sperm, const int *__restrict__ sdst,
               const real_t *__restrict__ x, const real_t *__restrict__ Y, const real_t *__restrict__ W,
               real_t *__restrict__ out, int n_nodes) {
    if ((int)blockIdx.x >= n_nodes) return;
    const int w = uni(threadIdx.x >> 6);
    const int grp = w / UCH, uc = w - grp * UCH;
    fwd_sender_dispatch<0>(grp, blockIdx.x, uc * 64 + (threadIdx.x & 63), srowptr, sperm, sdst, x, Y, W, out);
}

// m-major -> u-major inside each output block of one node row
extern "C" __global__ void __launch_bounds__(256)
oeq_out_untranspose(real_t *__restrict__ out) {
    __shared__ real_t t[OUT_BLOCK_MAX];
    g_untranspose_out_row(t, out + (i64)blockIdx.x * OD);
}

// Y-gradient flush of the sender-stationary VJP: row j of the tile belongs to edge sperm[base + j]
__device__ __forceinline__ void gy_flush_perm(GyStage &st, real_t *__restrict__ gY, const int *__restrict__ sperm,
                                              int base, int n) {
    if (UCH == 1) return;
    __syncthreads();
    for (int k = threadIdx.x; k < n * YD; k += UCH * 64) {
        const int j = k / YD, m = k - j * YD;
        real_t v = st.red[0][j][m];
#pragma unroll
        for (int w = 1; w < UCH; ++w) v += st.red[w][j][m];
        gY[(i64)sperm[base + j] * YD + m] = v;
    }
    __syncthreads();
}

// flags: bit0 store grad_W, bit1 store grad_Y, bit2 store grad_x
template <int G>
__device__ __forceinline__ void bwd_sender_group(GyStage &st, int s, int wv, int u, const int *__restrict__ srowptr,
                                                 const int *__restrict__ sperm, const int *__restrict__ sdst,
                                                 const real_t *__restrict__ x, const real_t *__restrict__ Y,
                                                 const real_t *__restrict__ W, const real_t *__restrict__ g,
                                                 real_t *__restrict__ gx, real_t *__restrict__ gY,
                                                 real_t *__restrict__ gW, int flags) {
    using Gr = BG<G>;
    const int lane = threadIdx.x & 63;
    const bool act = (U % 64 == 0) || (u < U);
    const int uu = act ? u : 0;
    const bool want_gw = (flags & 1) != 0, want_gy = (flags & 2) != 0, want_gx = (flags & 4) != 0;
    real_t xv[Gr::NX], gxa[Gr::NX];
    Gr::load_x(x + (i64)s * XD, uu, xv);
    if (!act) zero(xv);  // inactive lanes contribute nothing to the lane sums
    zero(gxa);
    const int k0 = uni(srowptr[s]), k1 = uni(srowptr[s + 1]);
    if (k0 < k1) {
        int e = uni(sperm[k0]), r = uni(sdst[k0]);
        real_t yv[YD], wv_[Gr::NW], gv[Gr::NO];
        load_y(Y, e, yv);
        Gr::load_w(W + (i64)e * (P * U), uu, wv_);
        Gr::load_g(g + (i64)r * OD, uu, gv);
        // the next edge's g row is prefetched only when it is small: it doubles the g registers
        constexpr bool PREF_G = Gr::NO <= 64;
        for (int k = k0; k < k1; ++k) {
            const int kn = (k + 1 < k1) ? k + 1 : k;
            const int en = uni(sperm[kn]), rn = uni(sdst[kn]);
            real_t yn[YD], wn[Gr::NW], gn[PREF_G ? Gr::NO : 1];
            load_y(Y, en, yn);
            Gr::load_w(W + (i64)en * (P * U), uu, wn);
            if constexpr (PREF_G) Gr::load_g(g + (i64)rn * OD, uu, gn);
            PIN_BWD();
            const int j = uni((k - k0) % GY_TILE);
            real_t gw[Gr::NW], gy[YD];
            zero(gw);
            zero(gy);
            Gr::template vjp<true, true, true>(xv, yv, wv_, gv, gw, gy, gxa);
            if (want_gw && act) Gr::store_w(gW + (i64)e * (P * U), u, gw);
            if (want_gy) {
                gy_push(st, gY, e, j, gy, lane, wv);
                if (j == GY_TILE - 1 || k + 1 == k1) gy_flush_perm(st, gY, sperm, k - j, j + 1);
            }
            e = en;
            r = rn;
#pragma unroll
            for (int q = 0; q < YD; ++q) yv[q] = yn[q];
#pragma unroll
            for (int q = 0; q < Gr::NW; ++q) wv_[q] = wn[q];
            if constexpr (PREF_G) {
#pragma unroll
                for (int q = 0; q < Gr::NO; ++q) gv[q] = gn[q];
            } else if (k + 1 < k1) {
                Gr::load_g(g + (i64)r * OD, uu, gv);
            }
        }
    }
    if (want_gx && act) Gr::store_x(gx + (i64)s * XD, u, gxa);
}

template <int G>
__device__ __forceinline__ void bwd_sender_dispatch(GyStage &st, int s, int grp, int wv, int u,
                                                    const int *__restrict__ srowptr, const int *__restrict__ sperm,
                                                    const int *__restrict__ sdst, const real_t *__restrict__ x,
                                                    const real_t *__restrict__ Y, const real_t *__restrict__ W,
                                                    const real_t *__restrict__ g, real_t *__restrict__ gx,
                                                    real_t *__restrict__ gY, real_t *__restrict__ gW, int flags) {
    if (grp == G) {
        bwd_sender_group<G>(st, s, wv, u, srowptr, sperm, sdst, x, Y, W, g, gx, gY, gW, flags);
        return;
    }
    if constexpr (G + 1 < NGB)
        bwd_sender_dispatch<G + 1>(st, s, grp, wv, u, srowptr, sperm, sdst, x, Y, W, g, gx, gY, gW, flags);
}

extern "C" __global__ void __launch_bounds__(UCH * 64) BWD_OCCUPANCY
oeq_bwd_sender(const int *__restrict__ srowptr, const int *__restrict__ sperm, const int *__restrict__ sdst,
               const real_t *__restrict__ x, const real_t *__restrict__ Y, const real_t *__restrict__ W,
               const real_t *__restrict__ g, real_t *__restrict__ gx, real_t *__restrict__ gY,
               real_t *__restrict__ gW, int flags, i64 gy_stride, int n_nodes) {
    __shared__ GyStage st;
    const int s = blockIdx.x / NGB, grp = blockIdx.x - s * NGB;
    if (s >= n_nodes) return;
    const int wv = uni(threadIdx.x >> 6);
    bwd_sender_dispatch<0>(st, s, grp, wv, wv * 64 + (threadIdx.x & 63), srowptr, sperm, sdst, x, Y, W, g, gx,
                           gY + grp * gy_stride, gW, flags);
}
