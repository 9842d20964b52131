// Kernel templates of the fused UVU CG tensor-product convolution (gfx950).
//
// The template is this file followed by kernels_conv, kernels_sender,
// kernels_gemm_radial, kernels_radial_fused and kernels_dbwd (in that order).
// It is compiled at plan time with hipRTC, after a prelude emitted by the
// planner that defines, for one descriptor and dtype: real_t; U, UCH (64-channel
// chunks), NGF / NGB / NGR (forward / backward / radial-backward path groups),
// P (paths), LY (largest Y degree), YD (Y row width), YSEL (the harmonic of degrees
// 0..LY behind each Y element), PY (YD rounded up to a power of two), LGPY
// (log2 PY), GY_TILE, XD, OD, XT; LDW / STW (loads and stores of W and its
// gradients); and the group structs FG<g> / BG<g> / RG<g> (see the planner's code
// generator) holding the unrolled sparse CG streams of one group of paths.
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

constexpr int YF = (LY + 1) * (LY + 1);  // harmonics of degrees 0..LY

__device__ __forceinline__ void sh_eval_full(real_t vx, real_t vy, real_t vz, real_t (&Yv)[YF]) {
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
__device__ __forceinline__ void sh_grad_full(real_t vx, real_t vy, real_t vz, const real_t (&gy)[YF], real_t &gvx,
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

// The plan's Y row from the harmonics of degrees 0..LY (the planner accepts vectors only
// for Y blocks of parity (-1)^l), and the gradient through it.
__device__ __forceinline__ void sh_eval(real_t vx, real_t vy, real_t vz, real_t (&Yv)[YD]) {
    real_t f[YF];
    sh_eval_full(vx, vy, vz, f);
#pragma unroll
    for (int k = 0; k < YD; ++k) Yv[k] = f[YSEL[k]];
}

__device__ __forceinline__ void sh_grad(real_t vx, real_t vy, real_t vz, const real_t (&gy)[YD], real_t &gvx,
                                        real_t &gvy, real_t &gvz) {
    real_t f[YF];
#pragma unroll
    for (int k = 0; k < YF; ++k) f[k] = real_t(0);
#pragma unroll
    for (int k = 0; k < YD; ++k) f[YSEL[k]] += gy[k];
    sh_grad_full(vx, vy, vz, f, gvx, gvy, gvz);
}

// Where a pass takes edge e's Y row from: YM_TENSOR the Y tensor, YM_VEC the harmonics
// of the edge vector vec[e], YM_POS the harmonics of pos[s] - pos[r] (the sender's
// position relative to the receiver; pr holds the receiver's position).
constexpr int YM_TENSOR = 0, YM_VEC = 1, YM_POS = 2;

template <int YM>
__device__ __forceinline__ void edge_y(const real_t *__restrict__ Ysrc, int e, int s, const real_t (&pr)[3],
                                       real_t (&yv)[YD]) {
    if constexpr (YM == YM_VEC) {
        const real_t *v = Ysrc + (i64)e * 3;
        sh_eval(v[0], v[1], v[2], yv);
    } else if constexpr (YM == YM_POS) {
        const real_t *ps = Ysrc + (i64)s * 3;
        sh_eval(ps[0] - pr[0], ps[1] - pr[1], ps[2] - pr[2], yv);
    } else {
        load_y(Ysrc, e, yv);
    }
}

// Edge vectors from positions, vec[e] = pos[src[e]] - pos[r], and their harmonics Y[e],
// one workgroup per receiver row r.
extern "C" __global__ void __launch_bounds__(64)
oeq_sph_harm_pos(const int *__restrict__ rowptr, const int *__restrict__ src, const real_t *__restrict__ pos,
                 real_t *__restrict__ Y, real_t *__restrict__ vec, int n_nodes) {
    const int r = blockIdx.x;
    if (r >= n_nodes) return;
    const real_t px = pos[(i64)r * 3], py = pos[(i64)r * 3 + 1], pz = pos[(i64)r * 3 + 2];
    const int e1 = rowptr[r + 1];
    for (int e = rowptr[r] + (int)threadIdx.x; e < e1; e += 64) {
        const i64 s = src[e];
        const real_t vx = pos[s * 3] - px, vy = pos[s * 3 + 1] - py, vz = pos[s * 3 + 2] - pz;
        vec[(i64)e * 3] = vx;
        vec[(i64)e * 3 + 1] = vy;
        vec[(i64)e * 3 + 2] = vz;
        real_t yv[YD];
        sh_eval(vx, vy, vz, yv);
#pragma unroll
        for (int k = 0; k < YD; ++k) Y[(i64)e * YD + k] = yv[k];
    }
}

// The position gradient from the edge-vector gradient gvec[E, 3]: each edge adds gvec[e]
// to its sender and subtracts it from its receiver (vec = pos[s] - pos[r]).  Atomic form:
// one workgroup per receiver row, gpos zeroed beforehand.
extern "C" __global__ void __launch_bounds__(64)
oeq_pos_scatter_atomic(const int *__restrict__ rowptr, const int *__restrict__ src, const real_t *__restrict__ gvec,
                       real_t *__restrict__ gpos, int n_nodes) {
    const int r = blockIdx.x;
    if (r >= n_nodes) return;
    const int e1 = rowptr[r + 1];
    for (int e = rowptr[r] + (int)threadIdx.x; e < e1; e += 64) {
        const i64 s = src[e];
#pragma unroll
        for (int c = 0; c < 3; ++c) {
            const real_t v = gvec[(i64)e * 3 + c];
            atomicAdd(gpos + s * 3 + c, v);
            atomicAdd(gpos + (i64)r * 3 + c, -v);
        }
    }
}

// Deterministic form: one thread per node n sums its out-edges in increasing edge id
// (the sender CSR) and then subtracts its own row's edges in order.
extern "C" __global__ void __launch_bounds__(256)
oeq_pos_scatter_det(const int *__restrict__ rowptr, const int *__restrict__ srowptr, const int *__restrict__ sperm,
                    const real_t *__restrict__ gvec, real_t *__restrict__ gpos, int n_nodes) {
    for (int n = blockIdx.x * blockDim.x + threadIdx.x; n < n_nodes; n += gridDim.x * blockDim.x) {
        real_t a0 = real_t(0), a1 = real_t(0), a2 = real_t(0);
        for (int k = srowptr[n]; k < srowptr[n + 1]; ++k) {
            const i64 e = sperm[k];
            a0 += gvec[e * 3];
            a1 += gvec[e * 3 + 1];
            a2 += gvec[e * 3 + 2];
        }
        for (int e = rowptr[n]; e < rowptr[n + 1]; ++e) {
            a0 -= gvec[(i64)e * 3];
            a1 -= gvec[(i64)e * 3 + 1];
            a2 -= gvec[(i64)e * 3 + 2];
        }
        gpos[(i64)n * 3] = a0;
        gpos[(i64)n * 3 + 1] = a1;
        gpos[(i64)n * 3 + 2] = a2;
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

// Sum of one value over the 64 lanes of a wave, in a fixed order; every lane gets it.
__device__ __forceinline__ real_t wave_sum(real_t v) {
    real_t a = v, b = v;
    swap32(a, b);
    v = a + b;
    a = v;
    b = v;
    swap16(a, b);
    v = a + b;
    v = v + dpp<kRor8>(v);
    v = v + xor4(v);
    v = v + dpp<kQxor2>(v);
    v = v + dpp<kQxor1>(v);
    return v;
}

extern "C" __global__ void __launch_bounds__(256)
oeq_fill_zero(real_t *__restrict__ p, i64 n) {
    for (i64 i = (i64)blockIdx.x * blockDim.x + threadIdx.x; i < n; i += (i64)gridDim.x * blockDim.x)
        p[i] = real_t(0);
}
