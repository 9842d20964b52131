// Kernel templates of the fused UVU CG tensor-product convolution (gfx950).
//
// This text is compiled at plan time with hipRTC, after a prelude emitted by
// the planner that defines, for one descriptor and dtype: real_t; U, UCH
// (64-channel chunks), NGF / NGB (forward / backward path groups), P (paths), YD
// ((L+1)^2), PY (YD rounded up to a power of two), LGPY (log2 PY), GY_TILE, XD,
// OD, XT; LDW / STW (loads and stores of W and its gradients); and the group
// structs FG<g> / BG<g> (see the planner's code generator) holding the unrolled
// sparse CG streams of one group of paths.
//
// Ownership follows "Receiver-streaming convolutions for channel-wise UVU tensor
// products" (opening post): a workgroup owns one receiver; each of its waves owns
// one 64-channel chunk (lane = channel) of one path group and streams the
// receiver's edges in CSR order.  The forward keeps its output values in
// registers and stores them once (no atomics).  The backward passes treat one
// edge at a time per wave: W-gradients are stored directly, Y-gradients are
// reduced across the 64 lanes and then across the waves through LDS, and
// x-gradients go to the senders either by hardware atomics or as per-edge rows
// summed later per sender.

__device__ __forceinline__ int uni(int v) { return __builtin_amdgcn_readfirstlane(v); }

template <int N>
__device__ __forceinline__ void zero(real_t (&a)[N]) {
#pragma unroll
    for (int i = 0; i < N; ++i) a[i] = real_t(0);
}

// Y row of edge e (wave-uniform: scalar loads).
__device__ __forceinline__ void load_y(const real_t *__restrict__ Y, int e, real_t (&yv)[YD]) {
    const real_t *yr = Y + (i64)e * YD;
#pragma unroll
    for (int k = 0; k < YD; ++k) yv[k] = yr[k];
}

// ---------------------------------------------------------------------------
// Real spherical harmonics of an edge vector v (degrees 0..LY, m = -l..l, l = 1
// ordered (y, z, x), component normalisation: the squares of degree l sum to
// 2l+1), evaluated on the direction n = v/|v| from the Cartesian polynomial forms
// of the Condon-Shortley real harmonics.  A zero vector has no direction: it
// gives Y_00 = 1 and zeros, and a zero gradient.
// ---------------------------------------------------------------------------
__device__ __forceinline__ float sqrt_r(float v) { return __builtin_sqrtf(v); }
__device__ __forceinline__ double sqrt_r(double v) { return __builtin_sqrt(v); }
__device__ __forceinline__ real_t rsqrt_or_zero(real_t r2) {
    return r2 > real_t(0) ? real_t(1) / sqrt_r(r2) : real_t(0);
}

__device__ __forceinline__ void sh_eval(real_t vx, real_t vy, real_t vz, real_t (&Yv)[YD]) {
    const real_t inv = rsqrt_or_zero(vx * vx + vy * vy + vz * vz);
    const real_t x = vx * inv, y = vy * inv, z = vz * inv;
    const bool live = inv > real_t(0);
    Yv[0] = real_t(1);
    if constexpr (LY >= 1) {
        const real_t s3 = real_t(1.7320508075688772);  // sqrt(3)
        Yv[1] = s3 * y;
        Yv[2] = s3 * z;
        Yv[3] = s3 * x;
    }
    if constexpr (LY >= 2) {
        const real_t s15 = real_t(3.872983346207417), s5 = real_t(2.23606797749979);
        Yv[4] = s15 * x * y;
        Yv[5] = s15 * y * z;
        Yv[6] = live ? real_t(0.5) * s5 * (real_t(3) * z * z - real_t(1)) : real_t(0);
        Yv[7] = s15 * x * z;
        Yv[8] = real_t(0.5) * s15 * (x * x - y * y);
    }
    if constexpr (LY >= 3) {
        const real_t a = real_t(2.091650066335189);   // sqrt(35/8)
        const real_t b = real_t(10.246950765959598);  // sqrt(105)
        const real_t c = real_t(1.6201851746019651);  // sqrt(21/8)
        const real_t h7 = real_t(1.3228756555322954); // sqrt(7)/2
        const real_t zz5 = real_t(5) * z * z - real_t(1);
        Yv[9] = a * y * (real_t(3) * x * x - y * y);
        Yv[10] = b * x * y * z;
        Yv[11] = c * y * zz5;
        Yv[12] = h7 * z * (real_t(5) * z * z - real_t(3));
        Yv[13] = c * x * zz5;
        Yv[14] = real_t(0.5) * b * z * (x * x - y * y);
        Yv[15] = a * x * (x * x - real_t(3) * y * y);
    }
}

// Vector gradient of sum_m gy[m] Y_m(v): with P_m the Cartesian polynomials above
// (any smooth extension off the sphere), grad = (I - n n^T) (sum_m gy[m] grad P_m(n)) / |v|.
__device__ __forceinline__ void sh_grad(real_t vx, real_t vy, real_t vz, const real_t (&gy)[YD], real_t &gvx,
                                        real_t &gvy, real_t &gvz) {
    const real_t inv = rsqrt_or_zero(vx * vx + vy * vy + vz * vz);
    const real_t x = vx * inv, y = vy * inv, z = vz * inv;
    real_t ax = real_t(0), ay = real_t(0), az = real_t(0);
    if constexpr (LY >= 1) {
        const real_t s3 = real_t(1.7320508075688772);
        ax += s3 * gy[3];
        ay += s3 * gy[1];
        az += s3 * gy[2];
    }
    if constexpr (LY >= 2) {
        const real_t s15 = real_t(3.872983346207417), s5 = real_t(2.23606797749979);
        // d/d(x,y,z) of s15 xy, s15 yz, s5/2 (3z^2-1), s15 xz, s15/2 (x^2-y^2)
        ax += s15 * (gy[4] * y + gy[7] * z + gy[8] * x);
        ay += s15 * (gy[4] * x + gy[5] * z - gy[8] * y);
        az += s15 * (gy[5] * y + gy[7] * x) + real_t(3) * s5 * gy[6] * z;
    }
    if constexpr (LY >= 3) {
        const real_t a = real_t(2.091650066335189), b = real_t(10.246950765959598);
        const real_t c = real_t(1.6201851746019651), h7 = real_t(1.3228756555322954);
        const real_t zz5 = real_t(5) * z * z - real_t(1);
        // a y(3x^2-y^2): (6a xy, 3a(x^2-y^2), 0)      b xyz: (b yz, b xz, b xy)
        // c y(5z^2-1): (0, c(5z^2-1), 10c yz)         sqrt(7)/2 (5z^3-3z): (0, 0, sqrt(7)/2 (15z^2-3))
        // c x(5z^2-1): (c(5z^2-1), 0, 10c xz)         b/2 z(x^2-y^2): (b xz, -b yz, b/2 (x^2-y^2))
        // a x(x^2-3y^2): (3a(x^2-y^2), -6a xy, 0)
        const real_t d2 = x * x - y * y;
        ax += real_t(6) * a * x * y * gy[9] + b * y * z * gy[10] + c * zz5 * gy[13] + b * x * z * gy[14] +
              real_t(3) * a * d2 * gy[15];
        ay += real_t(3) * a * d2 * gy[9] + b * x * z * gy[10] + c * zz5 * gy[11] - b * y * z * gy[14] -
              real_t(6) * a * x * y * gy[15];
        az += b * x * y * gy[10] + real_t(10) * c * y * z * gy[11] +
              h7 * (real_t(15) * z * z - real_t(3)) * gy[12] + real_t(10) * c * x * z * gy[13] +
              real_t(0.5) * b * d2 * gy[14];
    }
    const real_t dot = ax * x + ay * y + az * z;
    gvx = (ax - dot * x) * inv;
    gvy = (ay - dot * y) * inv;
    gvz = (az - dot * z) * inv;
}

// Y row of edge e from its vector (YV) or from memory
template <bool YV>
__device__ __forceinline__ void edge_y(const real_t *__restrict__ Ysrc, int e, real_t (&yv)[YD]) {
    if constexpr (YV) {
        const real_t *v = Ysrc + (i64)e * 3;
        sh_eval(v[0], v[1], v[2], yv);
    } else {
        load_y(Ysrc, e, yv);
    }
}

extern "C" __global__ void __launch_bounds__(256)
oeq_sph_harm(const real_t *__restrict__ vec, real_t *__restrict__ Y, i64 n_edges) {
    for (i64 e = (i64)blockIdx.x * blockDim.x + threadIdx.x; e < n_edges; e += (i64)gridDim.x * blockDim.x) {
        real_t yv[YD];
        sh_eval(vec[e * 3], vec[e * 3 + 1], vec[e * 3 + 2], yv);
#pragma unroll
        for (int k = 0; k < YD; ++k) Y[e * YD + k] = yv[k];
    }
}

extern "C" __global__ void __launch_bounds__(256)
oeq_sph_harm_bwd(const real_t *__restrict__ vec, const real_t *__restrict__ gY, real_t *__restrict__ gvec,
                 i64 n_edges) {
    for (i64 e = (i64)blockIdx.x * blockDim.x + threadIdx.x; e < n_edges; e += (i64)gridDim.x * blockDim.x) {
        real_t g[YD];
#pragma unroll
        for (int k = 0; k < YD; ++k) g[k] = gY[e * YD + k];
        real_t a, b, c;
        sh_grad(vec[e * 3], vec[e * 3 + 1], vec[e * 3 + 2], g, a, b, c);
        gvec[e * 3] = a;
        gvec[e * 3 + 1] = b;
        gvec[e * 3 + 2] = c;
    }
}

// Cross-lane moves on 32-bit words; a double moves as two words.
//   swap32(a, b): a <- [a lanes 0-31 | b lanes 0-31], b <- [a lanes 32-63 | b lanes 32-63]
//   swap16(a, b): per 32-lane half, a <- [a row 0 | b row 0], b <- [a row 1 | b row 1]
//   (v_permlane32_swap / v_permlane16_swap; rows are 16 lanes)
//   ror8: rotate by 8 inside each 16-lane row (the partner lane^8), DPP row_ror:8
//   xor4: the value of lane^4 (ds_swizzle, bit mode, xor mask 4)
//   qxor2 / qxor1: the value of lane^2 / lane^1 (DPP quad_perm)
__device__ __forceinline__ unsigned lo32(double v) { return (unsigned)(__double_as_longlong(v) & 0xffffffffull); }
__device__ __forceinline__ unsigned hi32(double v) { return (unsigned)(__double_as_longlong(v) >> 32); }
__device__ __forceinline__ double mk64(unsigned lo, unsigned hi) {
    return __longlong_as_double((long long)(((unsigned long long)hi << 32) | lo));
}
__device__ __forceinline__ void swap32(float &a, float &b) {
    auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(a), __float_as_uint(b), false, false);
    a = __uint_as_float(r[0]);
    b = __uint_as_float(r[1]);
}
__device__ __forceinline__ void swap32(double &a, double &b) {
    auto l = __builtin_amdgcn_permlane32_swap(lo32(a), lo32(b), false, false);
    auto h = __builtin_amdgcn_permlane32_swap(hi32(a), hi32(b), false, false);
    a = mk64(l[0], h[0]);
    b = mk64(l[1], h[1]);
}
__device__ __forceinline__ void swap16(float &a, float &b) {
    auto r = __builtin_amdgcn_permlane16_swap(__float_as_uint(a), __float_as_uint(b), false, false);
    a = __uint_as_float(r[0]);
    b = __uint_as_float(r[1]);
}
__device__ __forceinline__ void swap16(double &a, double &b) {
    auto l = __builtin_amdgcn_permlane16_swap(lo32(a), lo32(b), false, false);
    auto h = __builtin_amdgcn_permlane16_swap(hi32(a), hi32(b), false, false);
    a = mk64(l[0], h[0]);
    b = mk64(l[1], h[1]);
}
template <int CTRL>
__device__ __forceinline__ float dpp(float v) {
    return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), CTRL, 0xF, 0xF, false));
}
template <int CTRL>
__device__ __forceinline__ double dpp(double v) {
    return mk64((unsigned)__builtin_amdgcn_update_dpp(0, (int)lo32(v), CTRL, 0xF, 0xF, false),
                (unsigned)__builtin_amdgcn_update_dpp(0, (int)hi32(v), CTRL, 0xF, 0xF, false));
}
__device__ __forceinline__ float xor4(float v) { return __int_as_float(__builtin_amdgcn_ds_swizzle(__float_as_int(v), 0x101F)); }
__device__ __forceinline__ double xor4(double v) {
    return mk64((unsigned)__builtin_amdgcn_ds_swizzle((int)lo32(v), 0x101F),
                (unsigned)__builtin_amdgcn_ds_swizzle((int)hi32(v), 0x101F));
}
constexpr int kRor8 = 0x128, kQxor2 = 0x4E, kQxor1 = 0xB1;

// Sum of PY values over the 64 lanes of a wave, in a fixed order.  On return,
// lane l holds in v[0] the total of value (l >> (6 - LGPY)); every lane whose
// low (6 - LGPY) bits are zero may write it.  The first LGPY steps halve the
// values held per lane (at lane distances 32, 16, 8, 4: each lane keeps the half
// its distance bit selects and adds its partner's copy of that half); the other
// steps are plain butterflies over the remaining distances.
__device__ __forceinline__ void wave_reduce_scatter(real_t (&v)[PY], int lane) {
    if constexpr (LGPY >= 1) {
        constexpr int h = PY / 2;
#pragma unroll
        for (int i = 0; i < h; ++i) {
            real_t a = v[i], b = v[i + h];
            swap32(a, b);
            v[i] = a + b;
        }
    } else {
        real_t a = v[0], b = v[0];
        swap32(a, b);
        v[0] = a + b;
    }
    if constexpr (LGPY >= 2) {
        constexpr int h = PY / 4;
#pragma unroll
        for (int i = 0; i < h; ++i) {
            real_t a = v[i], b = v[i + h];
            swap16(a, b);
            v[i] = a + b;
        }
    } else {
        real_t a = v[0], b = v[0];
        swap16(a, b);
        v[0] = a + b;
    }
    if constexpr (LGPY >= 3) {
        constexpr int h = PY / 8;
        const bool up = (lane & 8) != 0;
#pragma unroll
        for (int i = 0; i < h; ++i) {
            const real_t s0 = v[i] + dpp<kRor8>(v[i]);
            const real_t s1 = v[i + h] + dpp<kRor8>(v[i + h]);
            v[i] = up ? s1 : s0;
        }
    } else {
        v[0] = v[0] + dpp<kRor8>(v[0]);
    }
    if constexpr (LGPY >= 4) {
        const bool up = (lane & 4) != 0;
        const real_t s0 = v[0] + xor4(v[0]);
        const real_t s1 = v[1] + xor4(v[1]);
        v[0] = up ? s1 : s0;
    } else {
        v[0] = v[0] + xor4(v[0]);
    }
    v[0] = v[0] + dpp<kQxor2>(v[0]);
    v[0] = v[0] + dpp<kQxor1>(v[0]);
}

extern "C" __global__ void __launch_bounds__(256)
oeq_fill_zero(real_t *__restrict__ p, i64 n) {
    for (i64 i = (i64)blockIdx.x * blockDim.x + threadIdx.x; i < n; i += (i64)gridDim.x * blockDim.x)
        p[i] = real_t(0);
}

// ---------------------------------------------------------------------------
// Forward: out[r] = sum over the receiver's edges of the per-edge messages.
// ---------------------------------------------------------------------------
template <int G, bool YV>
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
        // software pipeline: the next edge's loads are in flight while this one computes
        int s = uni(src[e0]);
        real_t yv[YD], xv[Gr::NX], wv[Gr::NW];
        edge_y<YV>(Y, e0, yv);
        Gr::load_x(x + (i64)s * XD, uu, xv);
        Gr::load_w(W + (i64)e0 * (P * U), uu, wv);
        for (int e = e0; e < e1; ++e) {
            real_t yn[YD], xn[Gr::NX], wn[Gr::NW];
            const int en = (e + 1 < e1) ? e + 1 : e;
            const int sn = uni(src[en]);
            edge_y<YV>(Y, en, yn);
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
}

template <int G, bool YV>
__device__ __forceinline__ void fwd_dispatch(int grp, int r, int u, const int *__restrict__ rowptr,
                                             const int *__restrict__ src, const real_t *__restrict__ x,
                                             const real_t *__restrict__ Y, const real_t *__restrict__ W,
                                             real_t *__restrict__ out, bool acc) {
    if (grp == G) {
        fwd_group<G, YV>(r, u, rowptr, src, x, Y, W, out, acc);
        return;
    }
    if constexpr (G + 1 < NGF) fwd_dispatch<G + 1, YV>(grp, r, u, rowptr, src, x, Y, W, out, acc);
}

extern "C" __global__ void __launch_bounds__(UCH * NGF * 64) FWD_OCCUPANCY
oeq_fwd(const int *__restrict__ rowptr, const int *__restrict__ src, const real_t *__restrict__ x,
        const real_t *__restrict__ Y, const real_t *__restrict__ W, real_t *__restrict__ out, int flags) {
    // flags: bit0 add into out instead of overwriting it
    const int w = uni(threadIdx.x >> 6);
    const int grp = w / UCH, uc = w - grp * UCH;
    fwd_dispatch<0, false>(grp, blockIdx.x, uc * 64 + (threadIdx.x & 63), rowptr, src, x, Y, W, out,
                           (flags & 1) != 0);
}

// The forward with Y evaluated in the kernel from the edge vectors vec[E, 3]
// (no Y tensor): each wave computes the harmonics of the edge it streams.
extern "C" __global__ void __launch_bounds__(UCH * NGF * 64) FWD_OCCUPANCY
oeq_fwd_vec(const int *__restrict__ rowptr, const int *__restrict__ src, const real_t *__restrict__ x,
            const real_t *__restrict__ vec, const real_t *__restrict__ W, real_t *__restrict__ out) {
    const int w = uni(threadIdx.x >> 6);
    const int grp = w / UCH, uc = w - grp * UCH;
    fwd_dispatch<0, true>(grp, blockIdx.x, uc * 64 + (threadIdx.x & 63), rowptr, src, x, vec, W, out, false);
}

// The atomic x-gradient is accumulated m-major inside each x block (so the
// lanes of one atomic instruction address consecutive words); this restores the
// u-major row layout in place, one node row per workgroup.
extern "C" __global__ void __launch_bounds__(256)
oeq_x_untranspose(real_t *__restrict__ gx) {
    __shared__ real_t t[XT ? XD : 1];
    real_t *row = gx + (i64)blockIdx.x * XD;
    if (!XT) return;
    for (int i = threadIdx.x; i < XD; i += 256) t[i] = row[i];
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
    // software pipeline: the next edge's loads are in flight while this one computes
    int s = uni(src[e0]);
    real_t yv[YD], xv[Gr::NX], wv_[Gr::NW];
    load_y(Y, e0, yv);
    Gr::load_x(x + (i64)s * XD, uu, xv);
    Gr::load_w(W + (i64)e0 * (P * U), uu, wv_);
    for (int e = e0; e < e1; ++e) {
        const int en = (e + 1 < e1) ? e + 1 : e;
        const int sn = uni(src[en]);
        real_t yn[YD], xn[Gr::NX], wn[Gr::NW];
        load_y(Y, en, yn);
        Gr::load_x(x + (i64)sn * XD, uu, xn);
        Gr::load_w(W + (i64)en * (P * U), uu, wn);
        // keep the next edge's loads ahead of this edge's arithmetic
        PIN_BWD();
        const int j = uni((e - e0) % GY_TILE);
        real_t gw[Gr::NW], gy[YD], gxp[Gr::NX];
        zero(gw);
        zero(gy);
        zero(gxp);
        Gr::template vjp<true, true, (GXMODE != 0)>(xv, yv, wv_, gv, gw, gy, gxp);
        if (want_gw && act) Gr::store_w(gW + (i64)e * (P * U), u, gw);
        if (want_gy) {
            gy_push(st, gY, e, j, gy, lane, wv);
            if (j == GY_TILE - 1 || e + 1 == e1) gy_flush(st, gY, e - j, j + 1);
        }
        if (GXMODE == 1 && act) Gr::atomic_x(gx + (i64)s * XD, u, gxp);
        if (GXMODE == 2 && act) Gr::store_x(gx + (i64)e * XD, u, gxp);
        s = sn;
#pragma unroll
        for (int k = 0; k < YD; ++k) yv[k] = yn[k];
#pragma unroll
        for (int k = 0; k < Gr::NX; ++k) xv[k] = xn[k];
#pragma unroll
        for (int k = 0; k < Gr::NW; ++k) wv_[k] = wn[k];
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
                                         real_t *__restrict__ gW, int flags, i64 gy_stride) {
    __shared__ GyStage st;
    const int r = blockIdx.x / NGB, grp = blockIdx.x - r * NGB;
    const int wv = uni(threadIdx.x >> 6);
    bwd_dispatch<GXMODE, 0>(st, r, grp, wv, wv * 64 + (threadIdx.x & 63), rowptr, src, x, Y, W, g, gx,
                            gY + grp * gy_stride, gW, flags);
}

extern "C" __global__ void __launch_bounds__(UCH * 64) BWD_OCCUPANCY
oeq_bwd_nogx(const int *__restrict__ rowptr, const int *__restrict__ src, const real_t *__restrict__ x,
             const real_t *__restrict__ Y, const real_t *__restrict__ W, const real_t *__restrict__ g,
             real_t *__restrict__ gx, real_t *__restrict__ gY, real_t *__restrict__ gW, int flags, i64 gy_stride) {
    bwd_body<0>(rowptr, src, x, Y, W, g, gx, gY, gW, flags, gy_stride);
}

extern "C" __global__ void __launch_bounds__(UCH * 64) BWD_OCCUPANCY
oeq_bwd_atomic(const int *__restrict__ rowptr, const int *__restrict__ src, const real_t *__restrict__ x,
               const real_t *__restrict__ Y, const real_t *__restrict__ W, const real_t *__restrict__ g,
               real_t *__restrict__ gx, real_t *__restrict__ gY, real_t *__restrict__ gW, int flags, i64 gy_stride) {
    bwd_body<1>(rowptr, src, x, Y, W, g, gx, gY, gW, flags, gy_stride);
}

extern "C" __global__ void __launch_bounds__(UCH * 64) BWD_OCCUPANCY
oeq_bwd_rows(const int *__restrict__ rowptr, const int *__restrict__ src, const real_t *__restrict__ x,
             const real_t *__restrict__ Y, const real_t *__restrict__ W, const real_t *__restrict__ g,
             real_t *__restrict__ h, real_t *__restrict__ gY, real_t *__restrict__ gW, int flags, i64 gy_stride) {
    bwd_body<2>(rowptr, src, x, Y, W, g, h, gY, gW, flags, gy_stride);
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
// sender CSR's (increasing edge id) order.
// ---------------------------------------------------------------------------
extern "C" __global__ void __launch_bounds__(256)
oeq_sender_sum(const int *__restrict__ srowptr, const int *__restrict__ sperm,
               const real_t *__restrict__ h, real_t *__restrict__ gx, int n_nodes) {
    const int s = blockIdx.x;
    if (s >= n_nodes) return;
    const int k0 = uni(srowptr[s]), k1 = uni(srowptr[s + 1]);
    for (i64 c = threadIdx.x; c < XD; c += 256) {
        real_t acc = real_t(0);
        int k = k0;
        // eight rows in flight, added in edge order
        for (; k + 8 <= k1; k += 8) {
            real_t t[8];
#pragma unroll
            for (int j = 0; j < 8; ++j) t[j] = h[(i64)uni(sperm[k + j]) * XD + c];
#pragma unroll
            for (int j = 0; j < 8; ++j) acc += t[j];
        }
        for (; k < k1; ++k) acc += h[(i64)uni(sperm[k]) * XD + c];
        gx[(i64)s * XD + c] = acc;
    }
}

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
               real_t *__restrict__ out) {
    const int w = uni(threadIdx.x >> 6);
    const int grp = w / UCH, uc = w - grp * UCH;
    fwd_sender_dispatch<0>(grp, blockIdx.x, uc * 64 + (threadIdx.x & 63), srowptr, sperm, sdst, x, Y, W, out);
}

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
               real_t *__restrict__ out) {
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
                if (GXMODE == 1 && act) Gr::atomic_x(gx + (i64)s * XD, u, gxp);
                if (GXMODE == 2 && act) Gr::store_x(gx + (i64)e * XD, u, gxp);
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
        real_t *__restrict__ dh, real_t *__restrict__ dw2p, int flags, i64 gy_stride, i64 dh_stride) {  \
        __shared__ GyStage st, sth;                                                                     \
        const int r = blockIdx.x / NGR, grp = blockIdx.x - r * NGR;                                     \
        const int wv = uni(threadIdx.x >> 6);                                                           \
        bwd_radial_dispatch<GXMODE, 0>(st, sth, r, grp, wv, wv * 64 + (threadIdx.x & 63), rowptr, src, x, Y, \
                                       hid, W2, g, gx, gY + grp * gy_stride, dh + grp * dh_stride, dw2p,  \
                                       flags);                                                          \
    }
OEQ_BWD_RADIAL_KERNEL(oeq_bwd_radial_nogx, 0)
OEQ_BWD_RADIAL_KERNEL(oeq_bwd_radial_atomic, 1)
OEQ_BWD_RADIAL_KERNEL(oeq_bwd_radial_rows, 2)

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
               real_t *__restrict__ gW, int flags, i64 gy_stride) {
    __shared__ GyStage st;
    const int s = blockIdx.x / NGB, grp = blockIdx.x - s * NGB;
    const int wv = uni(threadIdx.x >> 6);
    bwd_sender_dispatch<0>(st, s, grp, wv, wv * 64 + (threadIdx.x & 63), srowptr, sperm, sdst, x, Y, W, g, gx,
                           gY + grp * gy_stride, gW, flags);
}

// ---------------------------------------------------------------------------
// Dense matrix products on the matrix cores (the radial-weight MLP).
//   C[M,N] = alpha op(A)[M,K] op(B)[K,N]   (row-major; op = identity or transpose)
// A workgroup of 4 waves owns a BM x BN tile of C (oeq_gemm_<BM>x<BN>, 64 or 128 each);
// each wave a quarter, as blocks of the 16x16x4 MFMA (v_mfma_f32_16x16x4f32 /
// v_mfma_f64_16x16x4f64).  K advances 32 at a time through LDS.  blockIdx.z splits K: split s covers
// [s*kchunk, (s+1)*kchunk) and writes its tile to C + s*split_stride; with more
// than one split, oeq_gemm_reduce adds the partial tiles in split order.
// Operand lanes: A[l%16][l/16], B[l/16][l%16]; result value v of lane l is row
// 4(l/16)+v (fp32) or l/16+4v (fp64), column l%16.
// ---------------------------------------------------------------------------
typedef float mfma_f4 __attribute__((ext_vector_type(4)));
typedef double mfma_d4 __attribute__((ext_vector_type(4)));
__device__ __forceinline__ mfma_f4 mfma16(float a, float b, mfma_f4 c) {
    return __builtin_amdgcn_mfma_f32_16x16x4f32(a, b, c, 0, 0, 0);
}
__device__ __forceinline__ mfma_d4 mfma16(double a, double b, mfma_d4 c) {
    return __builtin_amdgcn_mfma_f64_16x16x4f64(a, b, c, 0, 0, 0);
}
typedef real_t mfma_acc __attribute__((ext_vector_type(4)));
__device__ __forceinline__ int mfma_row(int l, int v) {
    return sizeof(real_t) == 4 ? 4 * (l >> 4) + v : (l >> 4) + 4 * v;
}

constexpr int GK = 32;

// Workgroup tile GBM x BN (64 or 128 each): 4 waves as 2 x 2, each (GBM/2) x (BN/2) in
// 16x16 blocks, K staged GK at a time through LDS with the next chunk's loads in registers.
template <int GBM, int BN>
__device__ __forceinline__ void gemm_body(int M, int N, int K, const real_t *__restrict__ A, i64 lda, int ta,
                                          const real_t *__restrict__ B, i64 ldb, int tb, real_t *__restrict__ C,
                                          i64 ldc, i64 split_stride, int kchunk, real_t alpha) {
    constexpr int BI = GBM / 32, BJ = BN / 32;           // 16x16 blocks per wave
    constexpr int LA = GBM * GK / 256, LB = BN * GK / 256;  // elements per thread per chunk
    __shared__ real_t As[GBM][GK + 1];
    __shared__ real_t Bs[GK][BN + 1];
    const int t = threadIdx.x, l = t & 63, w = t >> 6;
    const int m0 = blockIdx.y * GBM, n0 = blockIdx.x * BN;
    const int kb = blockIdx.z * kchunk, ke = min(K, kb + kchunk);
    C += (i64)blockIdx.z * split_stride;
    const int wr = (w >> 1) * (GBM / 2), wc = (w & 1) * (BN / 2);
    mfma_acc acc[BI][BJ];
#pragma unroll
    for (int i = 0; i < BI; ++i)
#pragma unroll
        for (int j = 0; j < BJ; ++j) acc[i][j] = mfma_acc{0, 0, 0, 0};
    real_t ra[LA], rb[LB];
    // consecutive threads walk the contiguous dimension of each stored operand
    auto a_at = [&](int q, int &m, int &k) {
        const int idx = t + q * 256;
        if (ta) { k = idx / GBM; m = idx % GBM; } else { m = idx / GK; k = idx % GK; }
    };
    auto b_at = [&](int q, int &n, int &k) {
        const int idx = t + q * 256;
        if (tb) { n = idx / GK; k = idx % GK; } else { k = idx / BN; n = idx % BN; }
    };
    auto fetch = [&](int k0) {
#pragma unroll
        for (int q = 0; q < LA; ++q) {
            int m, k;
            a_at(q, m, k);
            const int gm = m0 + m, gk = k0 + k;
            ra[q] = (gm < M && gk < ke) ? (ta ? A[(i64)gk * lda + gm] : A[(i64)gm * lda + gk]) : real_t(0);
        }
#pragma unroll
        for (int q = 0; q < LB; ++q) {
            int n, k;
            b_at(q, n, k);
            const int gn = n0 + n, gk = k0 + k;
            rb[q] = (gn < N && gk < ke) ? (tb ? B[(i64)gn * ldb + gk] : B[(i64)gk * ldb + gn]) : real_t(0);
        }
    };
    auto stash = [&]() {
#pragma unroll
        for (int q = 0; q < LA; ++q) {
            int m, k;
            a_at(q, m, k);
            As[m][k] = ra[q];
        }
#pragma unroll
        for (int q = 0; q < LB; ++q) {
            int n, k;
            b_at(q, n, k);
            Bs[k][n] = rb[q];
        }
    };
    if (kb < ke) fetch(kb);
    for (int k0 = kb; k0 < ke; k0 += GK) {
        stash();
        __syncthreads();
        if (k0 + GK < ke) fetch(k0 + GK);
#pragma unroll
        for (int kk = 0; kk < GK; kk += 4) {
            real_t a[BI], b[BJ];
#pragma unroll
            for (int i = 0; i < BI; ++i) a[i] = As[wr + 16 * i + (l & 15)][kk + (l >> 4)];
#pragma unroll
            for (int j = 0; j < BJ; ++j) b[j] = Bs[kk + (l >> 4)][wc + 16 * j + (l & 15)];
#pragma unroll
            for (int i = 0; i < BI; ++i)
#pragma unroll
                for (int j = 0; j < BJ; ++j) acc[i][j] = mfma16(a[i], b[j], acc[i][j]);
        }
        __syncthreads();
    }
#pragma unroll
    for (int i = 0; i < BI; ++i)
#pragma unroll
        for (int j = 0; j < BJ; ++j)
#pragma unroll
            for (int v = 0; v < 4; ++v) {
                const int gm = m0 + wr + 16 * i + mfma_row(l, v), gn = n0 + wc + 16 * j + (l & 15);
                if (gm < M && gn < N) C[(i64)gm * ldc + gn] = alpha * acc[i][j][v];
            }
}

#define OEQ_GEMM_KERNEL(BM, BN)                                                                            \
    extern "C" __global__ void __launch_bounds__(256) oeq_gemm_##BM##x##BN(                                \
        int M, int N, int K, const real_t *__restrict__ A, i64 lda, int ta, const real_t *__restrict__ B,  \
        i64 ldb, int tb, real_t *__restrict__ C, i64 ldc, i64 split_stride, int kchunk, real_t alpha) {    \
        gemm_body<BM, BN>(M, N, K, A, lda, ta, B, ldb, tb, C, ldc, split_stride, kchunk, alpha);           \
    }
OEQ_GEMM_KERNEL(64, 64)
OEQ_GEMM_KERNEL(64, 128)
OEQ_GEMM_KERNEL(128, 64)
OEQ_GEMM_KERNEL(128, 128)

// First stage of an ordered sum of many partial rows: part [rows, n] -> out
// [ceil(rows / 32), n], chunk c holding rows 32c .. 32c+31 added in order.
extern "C" __global__ void __launch_bounds__(256)
oeq_sum_row_chunks(const real_t *__restrict__ part, int rows, i64 n, real_t *__restrict__ out) {
    const i64 c = (i64)blockIdx.x * blockDim.x + threadIdx.x;
    if (c >= n) return;
    const int r0 = blockIdx.y * 32, r1 = min(rows, r0 + 32);
    real_t s = part[(i64)r0 * n + c];
    for (int r = r0 + 1; r < r1; ++r) s += part[(i64)r * n + c];
    out[(i64)blockIdx.y * n + c] = s;
}

extern "C" __global__ void __launch_bounds__(256)
oeq_gemm_reduce(const real_t *__restrict__ part, int splits, i64 split_stride, int M, int N,
                real_t *__restrict__ C, i64 ldc) {
    const i64 n = (i64)M * N;
    for (i64 i = (i64)blockIdx.x * blockDim.x + threadIdx.x; i < n; i += (i64)gridDim.x * blockDim.x) {
        const i64 m = i / N, c = i - m * N;
        real_t s = part[m * N + c];
        for (int q = 1; q < splits; ++q) s += part[(i64)q * split_stride + m * N + c];
        C[m * ldc + c] = s;
    }
}

// ---------------------------------------------------------------------------
// Radial weights from edge lengths (a stated reading; the pages realise them
// outside the kernels): r = |vec|, d = r / r_cut,
//   u(d) = 1 - 28 d^6 + 48 d^7 - 21 d^8 (d < 1, else 0)    polynomial cutoff, p = 6
//   B_n(r) = sqrt(2 / r_cut) sin(n pi r / r_cut) / r u(d),  n = 1..8
//   h = silu(B W1 / sqrt(8)),  W = h W2 / sqrt(H)   (the two products on the matrix cores)
// ---------------------------------------------------------------------------
constexpr int RNB = 8;
__device__ __forceinline__ float sin_r(float v) { return sinf(v); }
__device__ __forceinline__ double sin_r(double v) { return sin(v); }
__device__ __forceinline__ float cos_r(float v) { return cosf(v); }
__device__ __forceinline__ double cos_r(double v) { return cos(v); }
__device__ __forceinline__ float exp_r(float v) { return expf(v); }
__device__ __forceinline__ double exp_r(double v) { return exp(v); }

// B_n(r) and, when D, dB_n/dr
template <bool D>
__device__ __forceinline__ void radial_basis(real_t r, real_t rc, real_t (&Bv)[RNB], real_t (&dBv)[RNB]) {
    const real_t pi = real_t(3.141592653589793);
    const real_t c = sqrt_r(real_t(2) / rc);
    const real_t d = r / rc;
    real_t u = real_t(0), du = real_t(0);
    if (d < real_t(1)) {
        const real_t d2 = d * d, d3 = d2 * d, d6 = d3 * d3;
        u = real_t(1) - real_t(28) * d6 + real_t(48) * d6 * d - real_t(21) * d6 * d2;
        const real_t om = real_t(1) - d;
        du = real_t(-168) * d2 * d3 * om * om;  // -p(p+1)(p+2)/2 d^(p-1) (1-d)^2
    }
#pragma unroll
    for (int n = 0; n < RNB; ++n) {
        const real_t k = real_t(n + 1) * pi / rc;
        if (r > real_t(0)) {
            const real_t sn = sin_r(k * r), inv = real_t(1) / r;
            Bv[n] = c * sn * inv * u;
            if constexpr (D) {
                const real_t ds = (k * cos_r(k * r) - sn * inv) * inv;
                dBv[n] = c * (ds * u + sn * inv * du / rc);
            }
        } else {
            Bv[n] = c * k * u;  // the limit sin(kr)/r -> k
            if constexpr (D) dBv[n] = real_t(0);
        }
    }
}

extern "C" __global__ void __launch_bounds__(256)
oeq_radial_basis(const real_t *__restrict__ vec, real_t rc, real_t *__restrict__ Bout, i64 n_edges) {
    for (i64 e = (i64)blockIdx.x * blockDim.x + threadIdx.x; e < n_edges; e += (i64)gridDim.x * blockDim.x) {
        const real_t x = vec[e * 3], y = vec[e * 3 + 1], z = vec[e * 3 + 2];
        real_t Bv[RNB], unused[RNB];
        radial_basis<false>(sqrt_r(x * x + y * y + z * z), rc, Bv, unused);
#pragma unroll
        for (int n = 0; n < RNB; ++n) Bout[e * RNB + n] = Bv[n];
    }
}

// pre = B W1 / sqrt(8) for element (e, j); DPRE: dh[e,j] *= silu'(pre), else h[e,j] = silu(pre)
template <bool DPRE>
__device__ __forceinline__ void radial_hidden_body(const real_t *__restrict__ Bm, const real_t *__restrict__ W1,
                                                   int H, real_t *__restrict__ io, i64 n_edges) {
    const i64 n = n_edges * H;
    for (i64 i = (i64)blockIdx.x * blockDim.x + threadIdx.x; i < n; i += (i64)gridDim.x * blockDim.x) {
        const i64 e = i / H;
        const int j = (int)(i - e * H);
        real_t pre = real_t(0);
#pragma unroll
        for (int q = 0; q < RNB; ++q) pre = fmar(Bm[e * RNB + q], W1[q * H + j], pre);
        pre *= real_t(0.35355339059327373);  // 1/sqrt(8)
        const real_t sg = real_t(1) / (real_t(1) + exp_r(-pre));
        if constexpr (DPRE)
            io[i] *= sg * (real_t(1) + pre * (real_t(1) - sg));
        else
            io[i] = pre * sg;
    }
}

extern "C" __global__ void __launch_bounds__(256)
oeq_radial_hidden(const real_t *__restrict__ Bm, const real_t *__restrict__ W1, int H, real_t *__restrict__ h,
                  i64 n_edges) {
    radial_hidden_body<false>(Bm, W1, H, h, n_edges);
}

extern "C" __global__ void __launch_bounds__(256)
oeq_radial_dpre(const real_t *__restrict__ Bm, const real_t *__restrict__ W1, int H, real_t *__restrict__ dh,
                i64 n_edges) {
    radial_hidden_body<true>(Bm, W1, H, dh, n_edges);
}

// grad_vec[e] = (sum_n dB[e,n] dB_n/dr) vec / r
extern "C" __global__ void __launch_bounds__(256)
oeq_radial_gvec(const real_t *__restrict__ vec, real_t rc, const real_t *__restrict__ dB, real_t *__restrict__ gvec,
                i64 n_edges) {
    for (i64 e = (i64)blockIdx.x * blockDim.x + threadIdx.x; e < n_edges; e += (i64)gridDim.x * blockDim.x) {
        const real_t x = vec[e * 3], y = vec[e * 3 + 1], z = vec[e * 3 + 2];
        const real_t r = sqrt_r(x * x + y * y + z * z);
        real_t Bv[RNB], dBv[RNB];
        radial_basis<true>(r, rc, Bv, dBv);
        real_t dr = real_t(0);
#pragma unroll
        for (int n = 0; n < RNB; ++n) dr = fmar(dB[e * RNB + n], dBv[n], dr);
        const real_t s = r > real_t(0) ? dr / r : real_t(0);
        gvec[e * 3] = s * x;
        gvec[e * 3 + 1] = s * y;
        gvec[e * 3 + 2] = s * z;
    }
}

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
constexpr int DW = 1, DY = 2, DG = 4, DX = 8;

template <int TM, int OUT, int G>
__device__ __forceinline__ void dbwd_group(GyStage &st, int r, int wv, int u, const int *__restrict__ rowptr,
                                           const int *__restrict__ src, const real_t *__restrict__ x,
                                           const real_t *__restrict__ Y, const real_t *__restrict__ W,
                                           const real_t *__restrict__ g, const real_t *__restrict__ ggx,
                                           const real_t *__restrict__ ggY, const real_t *__restrict__ ggW,
                                           real_t *__restrict__ dx, real_t *__restrict__ dY,
                                           real_t *__restrict__ dW, real_t *__restrict__ dg, int flags) {
    using Gr = BG<G>;
    const int lane = threadIdx.x & 63;
    const bool act = (U % 64 == 0) || (u < U);
    const int uu = act ? u : 0;
    const bool want_dw = (OUT & DW) && (flags & 1) != 0, want_dy = (OUT & DY) && (flags & 2) != 0,
               want_dg = (OUT & DG) && (flags & 4) != 0;
    const int dxmode = (OUT & DX) ? (flags >> 3) & 3 : 0;
    // add into the outputs instead of overwriting (one pass per tangent)
    const bool acc_dw = (flags & 32) != 0, acc_dy = (flags & 64) != 0, acc_dg = (flags & 128) != 0,
               acc_h = (flags & 256) != 0;
    constexpr bool HAS_DX = (TM & 6) != 0 && (OUT & DX) != 0;
    constexpr bool GW_ = (OUT & DW) != 0, GY_ = (OUT & DY) != 0, GX_ = (OUT & DX) != 0;
    real_t gv[Gr::NO];
    Gr::load_g(g + (i64)r * OD, uu, gv);
    if (!act) zero(gv);
    real_t dgacc[(OUT & DG) ? Gr::NO : 1];
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
            if constexpr ((TM & 1) != 0) {
                if constexpr ((OUT & DG) != 0)
                    if (want_dg) Gr::edge(cur.tx, cur.y, cur.w, dgacc);
                if constexpr (GW_ || GY_) Gr::template vjp<GW_, GY_, false>(cur.tx, cur.y, cur.w, gv, dw, dy, dxp);
            }
            if constexpr ((TM & 2) != 0) {
                if constexpr ((OUT & DG) != 0)
                    if (want_dg) Gr::edge(cur.x, cur.ty, cur.w, dgacc);
                if constexpr (GW_ || GX_) Gr::template vjp<GW_, false, GX_>(cur.x, cur.ty, cur.w, gv, dw, dy, dxp);
            }
            if constexpr ((TM & 4) != 0) {
                if constexpr ((OUT & DG) != 0)
                    if (want_dg) Gr::edge(cur.x, cur.y, cur.tw, dgacc);
                if constexpr (GY_ || GX_) Gr::template vjp<false, GY_, GX_>(cur.x, cur.y, cur.tw, gv, dw, dy, dxp);
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
            if (HAS_DX && dxmode == 1 && act) Gr::atomic_x(dx + (i64)s * XD, u, dxp);
            if (HAS_DX && dxmode == 2 && act) {
                if (acc_h)
                    Gr::add_x(dx + (i64)e * XD, u, dxp);
                else
                    Gr::store_x(dx + (i64)e * XD, u, dxp);
            }
            s = sn;
            cur = nxt;
        }
    }
    if constexpr ((OUT & DG) != 0)
    if (want_dg && act) {
        if (acc_dg)
            Gr::add_out(dg + (i64)r * OD, u, dgacc);
        else
            Gr::store_out(dg + (i64)r * OD, u, dgacc);
    }
}

template <int TM, int OUT, int G>
__device__ __forceinline__ void dbwd_dispatch(GyStage &st, int r, int grp, int wv, int u, const int *__restrict__ rowptr,
                                              const int *__restrict__ src, const real_t *__restrict__ x,
                                              const real_t *__restrict__ Y, const real_t *__restrict__ W,
                                              const real_t *__restrict__ g, const real_t *__restrict__ ggx,
                                              const real_t *__restrict__ ggY, const real_t *__restrict__ ggW,
                                              real_t *__restrict__ dx, real_t *__restrict__ dY,
                                              real_t *__restrict__ dW, real_t *__restrict__ dg, int flags) {
    if (grp == G) {
        dbwd_group<TM, OUT, G>(st, r, wv, u, rowptr, src, x, Y, W, g, ggx, ggY, ggW, dx, dY, dW, dg, flags);
        return;
    }
    if constexpr (G + 1 < NGB)
        dbwd_dispatch<TM, OUT, G + 1>(st, r, grp, wv, u, rowptr, src, x, Y, W, g, ggx, ggY, ggW, dx, dY, dW, dg,
                                      flags);
}

template <int TM, int OUT>
__device__ __forceinline__ void dbwd_body(const int *__restrict__ rowptr, const int *__restrict__ src,
                                          const real_t *__restrict__ x, const real_t *__restrict__ Y,
                                          const real_t *__restrict__ W, const real_t *__restrict__ g,
                                          const real_t *__restrict__ ggx, const real_t *__restrict__ ggY,
                                          const real_t *__restrict__ ggW, real_t *__restrict__ dx,
                                          real_t *__restrict__ dY, real_t *__restrict__ dW,
                                          real_t *__restrict__ dg, int flags, i64 gy_stride) {
    __shared__ GyStage st;
    const int r = blockIdx.x / NGB, grp = blockIdx.x - r * NGB;
    const int wv = uni(threadIdx.x >> 6);
    dbwd_dispatch<TM, OUT, 0>(st, r, grp, wv, wv * 64 + (threadIdx.x & 63), rowptr, src, x, Y, W, g, ggx, ggY, ggW, dx,
                         dY + grp * gy_stride, dW, dg, flags);
}

// oeq_dbwd_<TM>: every output in one pass.  oeq_dbwd_<TM>_<OUT>: the passes of
// the split double backward (d_W; d_Y and d_x; d_grad_out is left to the
// forward kernel, one accumulating launch per tangent).
#define OEQ_DBWD_KERNEL(NAME, TM, OUT)                                                              \
    extern "C" __global__ void __launch_bounds__(UCH * 64) BWD_OCCUPANCY NAME(                      \
        const int *__restrict__ rowptr, const int *__restrict__ src, const real_t *__restrict__ x, \
        const real_t *__restrict__ Y, const real_t *__restrict__ W, const real_t *__restrict__ g,  \
        const real_t *__restrict__ ggx, const real_t *__restrict__ ggY,                            \
        const real_t *__restrict__ ggW, real_t *__restrict__ dx, real_t *__restrict__ dY,          \
        real_t *__restrict__ dW, real_t *__restrict__ dg, int flags, i64 gy_stride) {              \
        dbwd_body<TM, OUT>(rowptr, src, x, Y, W, g, ggx, ggY, ggW, dx, dY, dW, dg, flags, gy_stride); \
    }
OEQ_DBWD_KERNEL(oeq_dbwd_1, 1, 15)
OEQ_DBWD_KERNEL(oeq_dbwd_2, 2, 15)
OEQ_DBWD_KERNEL(oeq_dbwd_3, 3, 15)
OEQ_DBWD_KERNEL(oeq_dbwd_4, 4, 15)
OEQ_DBWD_KERNEL(oeq_dbwd_5, 5, 15)
OEQ_DBWD_KERNEL(oeq_dbwd_6, 6, 15)
OEQ_DBWD_KERNEL(oeq_dbwd_7, 7, 15)
// d_W = BW(gg_x,Y,g) + BW(x,gg_Y,g): reads no weights
OEQ_DBWD_KERNEL(oeq_dbwd_1_1, 1, 1)
OEQ_DBWD_KERNEL(oeq_dbwd_2_1, 2, 1)
OEQ_DBWD_KERNEL(oeq_dbwd_3_1, 3, 1)
// d_Y and d_x of several tangents in one pass over W and gg_W
OEQ_DBWD_KERNEL(oeq_dbwd_3_10, 3, 10)
OEQ_DBWD_KERNEL(oeq_dbwd_5_10, 5, 10)
OEQ_DBWD_KERNEL(oeq_dbwd_6_10, 6, 10)
OEQ_DBWD_KERNEL(oeq_dbwd_7_10, 7, 10)
// one tangent: d_Y = BY(gg_x,W,g); d_x = Bx(gg_Y,W,g); d_Y, d_x = BY(x,gg_W,g), Bx(Y,gg_W,g)
OEQ_DBWD_KERNEL(oeq_dbwd_1_2, 1, 2)
OEQ_DBWD_KERNEL(oeq_dbwd_2_8, 2, 8)
OEQ_DBWD_KERNEL(oeq_dbwd_4_10, 4, 10)
