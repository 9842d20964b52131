// Dense products on the matrix cores and the radial-weight network.

// ---------------------------------------------------------------------------
// Dense matrix products on the matrix cores (the radial-weight MLP).
//   C[M,N] = alpha op(A)[M,K] op(B)[K,N]   (row-major; op = identity or transpose)
// A workgroup of 4 waves owns a BM x BN tile of C (oeq_gemm_<BM>x<BN>_<TA><TB>, sides 64 or 128,
// TA / TB the transposed operands);
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
// TA / TB: A stored [K, M] / B stored [N, K] (transposed operands).
template <int GBM, int BN, bool TA, bool TB>
__device__ __forceinline__ void gemm_body(int M, int N, int K, const real_t *__restrict__ A, i64 lda,
                                          const real_t *__restrict__ B, i64 ldb, real_t *__restrict__ C,
                                          i64 ldc, i64 split_stride, int kchunk, real_t alpha) {
    constexpr int BI = GBM / 32, BJ = BN / 32;              // 16x16 blocks per wave
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
    // Consecutive threads walk the contiguous dimension of each stored operand.  Element q
    // of a thread sits at (row, k) = (am + q*AMS, ak + q*AKS) of the A tile and
    // (bk + q*BKS, bn + q*BNS) of the B tile: affine in q, so no per-element state.
    constexpr int AMS = TA ? 0 : 256 / GK, AKS = TA ? 256 / GBM : 0;
    constexpr int BKS = TB ? 0 : 256 / BN, BNS = TB ? 256 / GK : 0;
    const int am = TA ? t % GBM : t / GK, ak = TA ? t / GBM : t % GK;
    const int bn = TB ? t / GK : t % BN, bk = TB ? t % GK : t / BN;
    const i64 aoff = TA ? (i64)ak * lda + am : (i64)am * lda + ak;           // at q = 0
    const i64 aq = TA ? (i64)AKS * lda : (i64)AMS * lda;                       // per q
    const i64 boff = TB ? (i64)bn * ldb + bk : (i64)bk * ldb + bn;
    const i64 bq = TB ? (i64)BNS * ldb : (i64)BKS * ldb;
    real_t ra[LA], rb[LB];
    // Out-of-range elements read the chunk's first element (always valid); they are
    // zeroed when stashed, so the loads themselves carry no dependence and stay in flight.
    auto a_ok = [&](int q, int kl) { return (m0 + am + q * AMS < M) && (ak + q * AKS < kl); };
    auto b_ok = [&](int q, int kl) { return (n0 + bn + q * BNS < N) && (bk + q * BKS < kl); };
    auto fetch = [&](int k0) {
        const real_t *Ab = TA ? A + (i64)k0 * lda + m0 : A + (i64)m0 * lda + k0;
        const real_t *Bb = TB ? B + (i64)n0 * ldb + k0 : B + (i64)k0 * ldb + n0;
        const int kl = ke - k0;  // K values left in this chunk
#pragma unroll
        for (int q = 0; q < LA; ++q) ra[q] = Ab[a_ok(q, kl) ? aoff + q * aq : 0];
#pragma unroll
        for (int q = 0; q < LB; ++q) rb[q] = Bb[b_ok(q, kl) ? boff + q * bq : 0];
    };
    auto stash = [&](int k0) {
        const int kl = ke - k0;
#pragma unroll
        for (int q = 0; q < LA; ++q) As[am + q * AMS][ak + q * AKS] = a_ok(q, kl) ? ra[q] : real_t(0);
#pragma unroll
        for (int q = 0; q < LB; ++q) Bs[bk + q * BKS][bn + q * BNS] = b_ok(q, kl) ? rb[q] : real_t(0);
    };
    if (kb < ke) fetch(kb);
    for (int k0 = kb; k0 < ke; k0 += GK) {
        stash(k0);
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
    real_t *Ct = C + (i64)(m0 + wr) * ldc + n0 + wc + (l & 15);
    if (m0 + GBM <= M && n0 + BN <= N) {  // interior tile: no bounds tests
#pragma unroll
        for (int i = 0; i < BI; ++i)
#pragma unroll
            for (int j = 0; j < BJ; ++j)
#pragma unroll
                for (int v = 0; v < 4; ++v) Ct[(i64)(16 * i + mfma_row(l, v)) * ldc + 16 * j] = alpha * acc[i][j][v];
        return;
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

#define OEQ_GEMM_KERNEL(BM, BN, TA, TB)                                                                   \
    extern "C" __global__ void __launch_bounds__(256) oeq_gemm_##BM##x##BN##_##TA##TB(                    \
        int M, int N, int K, const real_t *__restrict__ A, i64 lda, const real_t *__restrict__ B, i64 ldb, \
        real_t *__restrict__ C, i64 ldc, i64 split_stride, int kchunk, real_t alpha) {                     \
        gemm_body<BM, BN, TA != 0, TB != 0>(M, N, K, A, lda, B, ldb, C, ldc, split_stride, kchunk, alpha); \
    }
#define OEQ_GEMM_SHAPES(TA, TB)          \
    OEQ_GEMM_KERNEL(64, 64, TA, TB)      \
    OEQ_GEMM_KERNEL(64, 128, TA, TB)     \
    OEQ_GEMM_KERNEL(128, 64, TA, TB)     \
    OEQ_GEMM_KERNEL(128, 128, TA, TB)
OEQ_GEMM_SHAPES(0, 0)
OEQ_GEMM_SHAPES(0, 1)
OEQ_GEMM_SHAPES(1, 0)

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
