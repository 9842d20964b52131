/*
 * CPU oracle for the fused channel-wise (UVU) Clebsch-Gordan tensor-product
 * graph convolution: forward, vector-Jacobian product and double backward.
 *
 * TEST INFRASTRUCTURE ONLY.  Only the test suite, the smoke check and the
 * benchmark's CPU-baseline leg may load this library.  The GPU library shares
 * no code, header, table or constant with it, and neither side calls the other.
 *
 * Everything is plain fp64 nested loops written from the definitions:
 *
 *  - Complex Clebsch-Gordan coefficients from Racah's closed form
 *    (Condon-Shortley phase).  The CG tensor product itself is described in
 *    "An Efficient Sparse Kernel Generator for O(3)-Equivariant Deep Networks"
 *    (abstract): two dense feature vectors contracted with a structured sparse
 *    tensor into a dense output.
 *  - Real-basis CG: the complex coefficients carried to the real spherical-
 *    harmonic basis by the unitary change of basis A_l, keeping the real or the
 *    imaginary part according to the parity of l1+l2+l3, then signed so that
 *    the first non-zero entry (row-major in m1, m2, m3) is positive; entries
 *    with magnitude <= 1e-10 are stored as exact zeros.
 *  - The channel-wise convolution of "Receiver-streaming convolutions for
 *    channel-wise UVU tensor products" (opening post): for every edge s->r,
 *    every path (l1, l2 -> l3) and every channel u,
 *        out[r,u,l3 m3] += sum_{m1,m2} C[m1,m2,m3] x[s,u,l1 m1] Y[e,l2 m2] W[e,p,u].
 *  - Its gradients with respect to x, Y and W (sums over the same terms), and
 *    the double backward through the identity that follows from the map being
 *    linear in each of x, Y and W separately (see oracle_dbwd below).
 *
 * OpenMP is used only over rows whose results are independent (receivers for
 * the forward, edges for the W and Y gradients, senders for the x gradient), so
 * every result is deterministic and independent of the thread count.
 *
 * Layouts (one convention, stated once):
 *   x  [N, XD]  block i (degree l_i, U channels) at xoff_i, element u*(2l_i+1)+(m+l_i)
 *   Y  [E, YD]  Y block j (degree l_j, one channel) at yoff_j = sum of (2l+1) over the
 *               blocks before it, element yoff_j + (m2+l_j); with the blocks 0e, 1o,
 *               2e, .. L this is element l2*l2 + (m2+l2)
 *   W  [E, P, U]
 *   out[N, OD]  output block o (degree l_o) at ooff_o, element u*(2l_o+1)+(m+l_o)
 * A block of multiplicity 1 (x or output) has one channel: element (m+l) at its
 * offset.  Channel u of a path reads channel u of its x block, or the single
 * channel of a multiplicity-1 x block (broadcast), and adds into channel u of its
 * output block, or into the single channel of a multiplicity-1 output block (a sum
 * over the channels): a UVW product whose weight is diagonal in (u, w) up to such a
 * broadcast or sum, which reduces to the channel-wise one.
 * Edge e lies in receiver row r when rowptr[r] <= e < rowptr[r+1]; its sender
 * is src[e].
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

#define ORACLE_LMAX 3
#define ORACLE_NM (2 * ORACLE_LMAX + 1)

/* ------------------------------------------------------------------ */
/* Complex Clebsch-Gordan coefficients: Racah's closed form.           */
/* ------------------------------------------------------------------ */

static double fact(int n) {
    double f = 1.0;
    for (int i = 2; i <= n; ++i) f *= (double)i;
    return f; /* exact in double for n <= 18 */
}

/* <j1 m1 j2 m2 | J M> for integer angular momenta. */
double oracle_cg_complex(int j1, int m1, int j2, int m2, int J, int M) {
    if (m1 + m2 != M) return 0.0;
    if (j1 < 0 || j2 < 0 || J < 0) return 0.0;
    if (abs(m1) > j1 || abs(m2) > j2 || abs(M) > J) return 0.0;
    if (J < abs(j1 - j2) || J > j1 + j2) return 0.0;
    double pre1 = (2.0 * J + 1.0) * fact(J + j1 - j2) * fact(J - j1 + j2) *
                  fact(j1 + j2 - J) / fact(j1 + j2 + J + 1);
    double pre2 = fact(J + M) * fact(J - M) * fact(j1 - m1) * fact(j1 + m1) *
                  fact(j2 - m2) * fact(j2 + m2);
    double sum = 0.0;
    for (int k = 0; k <= j1 + j2 + J; ++k) {
        int a[6] = {k, j1 + j2 - J - k, j1 - m1 - k, j2 + m2 - k,
                    J - j2 + m1 + k, J - j1 - m2 + k};
        int ok = 1;
        for (int t = 0; t < 6; ++t)
            if (a[t] < 0) ok = 0;
        if (!ok) continue;
        double den = 1.0;
        for (int t = 0; t < 6; ++t) den *= fact(a[t]);
        sum += ((k & 1) ? -1.0 : 1.0) / den;
    }
    return sqrt(pre1) * sqrt(pre2) * sum;
}

/* ------------------------------------------------------------------ */
/* Real basis: A_l[m][mu], rows real m, columns complex mu, both -l..l. */
/* ------------------------------------------------------------------ */

static void real_basis(int l, double re[ORACLE_NM][ORACLE_NM],
                       double im[ORACLE_NM][ORACLE_NM]) {
    const double h = 1.0 / sqrt(2.0);
    for (int a = 0; a < ORACLE_NM; ++a)
        for (int b = 0; b < ORACLE_NM; ++b) re[a][b] = im[a][b] = 0.0;
    for (int m = -l; m <= l; ++m) {
        int r = m + l;
        double sgn = (abs(m) & 1) ? -1.0 : 1.0; /* (-1)^m */
        if (m > 0) {
            re[r][m + l] = sgn * h;
            re[r][-m + l] = h;
        } else if (m == 0) {
            re[r][l] = 1.0;
        } else {
            im[r][m + l] = h;            /* A[m][m]   =  i/sqrt2          */
            im[r][-m + l] = -sgn * h;    /* A[m][|m|] = -i (-1)^m / sqrt2 */
        }
    }
}

/* Export of A_l for tests (row-major (2l+1)x(2l+1), real and imaginary parts). */
void oracle_real_basis(int l, double *re_out, double *im_out) {
    double re[ORACLE_NM][ORACLE_NM], im[ORACLE_NM][ORACLE_NM];
    real_basis(l, re, im);
    int n = 2 * l + 1;
    for (int a = 0; a < n; ++a)
        for (int b = 0; b < n; ++b) {
            re_out[a * n + b] = re[a][b];
            im_out[a * n + b] = im[a][b];
        }
}

/* Raw real-basis tensor T[m1,m2,m3] = sum conj(A1) conj(A2) A3 <l1 mu1 l2 mu2|l3 mu3>
 * (complex), before the choice of real/imaginary part and the sign canon.
 * Dense row-major over (m1+l1, m2+l2, m3+l3).  Returns 0, or -1 if l out of range. */
int oracle_cg_real_raw(int l1, int l2, int l3, double *t_re, double *t_im) {
    if (l1 < 0 || l2 < 0 || l3 < 0 || l1 > ORACLE_LMAX || l2 > ORACLE_LMAX ||
        l3 > ORACLE_LMAX)
        return -1;
    double a1r[ORACLE_NM][ORACLE_NM], a1i[ORACLE_NM][ORACLE_NM];
    double a2r[ORACLE_NM][ORACLE_NM], a2i[ORACLE_NM][ORACLE_NM];
    double a3r[ORACLE_NM][ORACLE_NM], a3i[ORACLE_NM][ORACLE_NM];
    real_basis(l1, a1r, a1i);
    real_basis(l2, a2r, a2i);
    real_basis(l3, a3r, a3i);
    int n1 = 2 * l1 + 1, n2 = 2 * l2 + 1, n3 = 2 * l3 + 1;
    for (int i = 0; i < n1; ++i)
        for (int j = 0; j < n2; ++j)
            for (int k = 0; k < n3; ++k) {
                double sr = 0.0, si = 0.0;
                for (int a = 0; a < n1; ++a)
                    for (int b = 0; b < n2; ++b)
                        for (int c = 0; c < n3; ++c) {
                            double cg = oracle_cg_complex(l1, a - l1, l2, b - l2,
                                                          l3, c - l3);
                            if (cg == 0.0) continue;
                            /* conj(A1[i,a]) * conj(A2[j,b]) */
                            double pr = a1r[i][a] * a2r[j][b] - a1i[i][a] * a2i[j][b];
                            double pi = -(a1r[i][a] * a2i[j][b] + a1i[i][a] * a2r[j][b]);
                            /* times A3[k,c] */
                            double qr = pr * a3r[k][c] - pi * a3i[k][c];
                            double qi = pr * a3i[k][c] + pi * a3r[k][c];
                            sr += qr * cg;
                            si += qi * cg;
                        }
                t_re[(i * n2 + j) * n3 + k] = sr;
                t_im[(i * n2 + j) * n3 + k] = si;
            }
    return 0;
}

/* Real-basis CG table C[m1,m2,m3] (dense, row-major), sign-canonical, with
 * entries of magnitude <= 1e-10 set to exactly zero.
 * Returns the number of non-zero entries, 0 if (l1,l2,l3) violates the
 * triangle rule, or -1 if an l is outside 0..3. */
int oracle_cg_real(int l1, int l2, int l3, double *C) {
    if (l1 < 0 || l2 < 0 || l3 < 0 || l1 > ORACLE_LMAX || l2 > ORACLE_LMAX ||
        l3 > ORACLE_LMAX)
        return -1;
    int n1 = 2 * l1 + 1, n2 = 2 * l2 + 1, n3 = 2 * l3 + 1, n = n1 * n2 * n3;
    if (l3 < abs(l1 - l2) || l3 > l1 + l2) {
        for (int i = 0; i < n; ++i) C[i] = 0.0;
        return 0;
    }
    double tre[ORACLE_NM * ORACLE_NM * ORACLE_NM], tim[ORACLE_NM * ORACLE_NM * ORACLE_NM];
    oracle_cg_real_raw(l1, l2, l3, tre, tim);
    const double *src = ((l1 + l2 + l3) % 2 == 0) ? tre : tim;
    double sign = 0.0;
    for (int i = 0; i < n; ++i)
        if (fabs(src[i]) > 1e-10) {
            sign = src[i] > 0 ? 1.0 : -1.0;
            break;
        }
    int nnz = 0;
    for (int i = 0; i < n; ++i) {
        double v = sign * src[i];
        if (fabs(v) > 1e-10) {
            C[i] = v;
            ++nnz;
        } else {
            C[i] = 0.0;
        }
    }
    return nnz;
}

/* ------------------------------------------------------------------ */
/* Path enumeration (all triangle-allowed outputs up to l3max).        */
/* ------------------------------------------------------------------ */

/* x blocks in descriptor order, then the Y blocks in their order, then
 * l3 = |l1-l2|..min(l1+l2, l3max), l2 the Y block's degree.  Output parity
 * p3 = p1 * pY (the product of the two inputs' parities).  Writes rows
 * (i1, Y block, l3, p3) into out[4*k]; returns the number of paths (or the number
 * that would be written, if larger than max_paths). */
int oracle_enumerate_paths_y(int nx, const int *xl, const int *xpar, int ny, const int *yl,
                             const int *ypar, int l3max, int *out, int max_paths) {
    int k = 0;
    for (int i = 0; i < nx; ++i)
        for (int j = 0; j < ny; ++j) {
            int l2 = yl[j];
            int lo = abs(xl[i] - l2), hi = xl[i] + l2;
            if (hi > l3max) hi = l3max;
            for (int l3 = lo; l3 <= hi; ++l3) {
                if (k < max_paths) {
                    out[4 * k + 0] = i;
                    out[4 * k + 1] = j;
                    out[4 * k + 2] = l3;
                    out[4 * k + 3] = xpar[i] * ypar[j];
                }
                ++k;
            }
        }
    return k;
}

/* The spherical harmonics of degrees 0..L as Y blocks (degree l, parity (-1)^l). */
int oracle_enumerate_paths(int nx, const int *xl, const int *xpar, int L,
                           int l3max, int *out, int max_paths) {
    int yl[ORACLE_LMAX + 1], ypar[ORACLE_LMAX + 1];
    if (L < 0 || L > ORACLE_LMAX) return 0;
    for (int l = 0; l <= L; ++l) {
        yl[l] = l;
        ypar[l] = (l & 1) ? -1 : 1;
    }
    return oracle_enumerate_paths_y(nx, xl, xpar, L + 1, yl, ypar, l3max, out, max_paths);
}

/* ------------------------------------------------------------------ */
/* Problem description and sparse per-path tables.                      */
/* ------------------------------------------------------------------ */

typedef struct {
    int nx;            /* number of x blocks                                */
    const int *xl;     /* degree of each x block (all with U channels)      */
    int U;             /* channels                                          */
    int ny;            /* number of Y blocks (one channel each)             */
    const int *yl;     /* degree of each Y block, in row order              */
    int np;            /* number of paths                                   */
    const int *p_i1;   /* x block of each path                              */
    const int *p_iy;   /* Y block of each path                              */
    const int *p_l3;   /* output degree of each path                        */
    const int *p_ob;   /* output block of each path                         */
    int nob;           /* number of output blocks                           */
    const int *ob_l;   /* degree of each output block                       */
    const int *xm;     /* channels of each x block: U, or 1 (NULL: all U)   */
    const int *om;     /* channels of each output block: U or 1 (NULL: U)   */
} oracle_desc;

typedef struct {
    int nnz;
    int m1[ORACLE_NM * ORACLE_NM * ORACLE_NM];
    int m2[ORACLE_NM * ORACLE_NM * ORACLE_NM];
    int m3[ORACLE_NM * ORACLE_NM * ORACLE_NM];
    double c[ORACLE_NM * ORACLE_NM * ORACLE_NM];
    int64_t xoff, ooff; /* block offsets within a node row                 */
    int n1, n2, n3;     /* 2l1+1, 2l2+1, 2l3+1                            */
    int xu, ou;         /* 1 when the x / output block has U channels, 0 for one channel */
    int yoff;           /* offset of the path's Y block in a Y row        */
} oracle_path;

/* Returns 0 on success, -1 on an invalid description.  Fills the per-path
 * tables and the row widths. */
static int build_paths(const oracle_desc *d, oracle_path *pt, int64_t *xd,
                       int64_t *od, int *yd) {
    if (d->nx <= 0 || d->U <= 0 || d->ny <= 0 || d->ny > 64 || d->np < 0 || d->nob < 0)
        return -1;
    int64_t xoff[64], ooff[64];
    int yoff[64];
    if (d->nx > 64 || d->nob > 64) return -1;
    int64_t acc = 0;
    for (int i = 0; i < d->nx; ++i) {
        if (d->xl[i] < 0 || d->xl[i] > ORACLE_LMAX) return -1;
        const int m = d->xm ? d->xm[i] : d->U;
        if (m != d->U && m != 1) return -1;
        xoff[i] = acc;
        acc += (int64_t)m * (2 * d->xl[i] + 1);
    }
    *xd = acc;
    acc = 0;
    for (int o = 0; o < d->nob; ++o) {
        if (d->ob_l[o] < 0 || d->ob_l[o] > ORACLE_LMAX) return -1;
        const int m = d->om ? d->om[o] : d->U;
        if (m != d->U && m != 1) return -1;
        ooff[o] = acc;
        acc += (int64_t)m * (2 * d->ob_l[o] + 1);
    }
    *od = acc;
    int ya = 0;
    for (int j = 0; j < d->ny; ++j) {
        if (d->yl[j] < 0 || d->yl[j] > ORACLE_LMAX) return -1;
        yoff[j] = ya;
        ya += 2 * d->yl[j] + 1;
    }
    *yd = ya;
    for (int p = 0; p < d->np; ++p) {
        int i1 = d->p_i1[p], iy = d->p_iy[p], l3 = d->p_l3[p], ob = d->p_ob[p];
        if (i1 < 0 || i1 >= d->nx || iy < 0 || iy >= d->ny || ob < 0 || ob >= d->nob)
            return -1;
        int l2 = d->yl[iy];
        if (d->ob_l[ob] != l3) return -1;
        int l1 = d->xl[i1];
        double C[ORACLE_NM * ORACLE_NM * ORACLE_NM];
        if (oracle_cg_real(l1, l2, l3, C) <= 0) return -1;
        int n1 = 2 * l1 + 1, n2 = 2 * l2 + 1, n3 = 2 * l3 + 1, k = 0;
        for (int a = 0; a < n1; ++a)
            for (int b = 0; b < n2; ++b)
                for (int c = 0; c < n3; ++c) {
                    double v = C[(a * n2 + b) * n3 + c];
                    if (v == 0.0) continue;
                    pt[p].m1[k] = a;
                    pt[p].m2[k] = b;
                    pt[p].m3[k] = c;
                    pt[p].c[k] = v;
                    ++k;
                }
        pt[p].nnz = k;
        pt[p].xoff = xoff[i1];
        pt[p].ooff = ooff[ob];
        pt[p].n1 = n1;
        pt[p].n2 = n2;
        pt[p].n3 = n3;
        pt[p].xu = (d->xm ? d->xm[i1] : d->U) == d->U;
        pt[p].ou = (d->om ? d->om[ob] : d->U) == d->U;
        pt[p].yoff = yoff[iy];
    }
    return 0;
}

/* Receiver of every edge, from the receiver CSR. */
static void edge_receivers(int64_t N, const int32_t *rowptr, int32_t *recv) {
    for (int64_t r = 0; r < N; ++r)
        for (int64_t e = rowptr[r]; e < rowptr[r + 1]; ++e) recv[e] = (int32_t)r;
}

/* ------------------------------------------------------------------ */
/* Sender CSR: counting sort of edges by sender, filled in increasing e. */
/* ------------------------------------------------------------------ */

void oracle_sender_csr(int64_t N, int64_t E, const int32_t *src, int32_t *srowptr,
                       int32_t *sperm) {
    for (int64_t s = 0; s <= N; ++s) srowptr[s] = 0;
    for (int64_t e = 0; e < E; ++e) srowptr[src[e] + 1] += 1;
    for (int64_t s = 0; s < N; ++s) srowptr[s + 1] += srowptr[s];
    int32_t *fill = (int32_t *)malloc(sizeof(int32_t) * (size_t)(N > 0 ? N : 1));
    for (int64_t s = 0; s < N; ++s) fill[s] = srowptr[s];
    for (int64_t e = 0; e < E; ++e) sperm[fill[src[e]]++] = (int32_t)e;
    free(fill);
}

/* ------------------------------------------------------------------ */
/* Forward.                                                             */
/* ------------------------------------------------------------------ */

/* out_rows[k, :] = out[rows[k], :] of the convolution f(x, Y, W).
 * rows == NULL means all N receivers in order (nrows must equal N). */
int oracle_fwd(const oracle_desc *d, int64_t N, int64_t E, const int32_t *rowptr,
               const int32_t *src, const double *x, const double *Y, const double *W,
               const int64_t *rows, int64_t nrows, double *out_rows) {
    oracle_path *pt = (oracle_path *)malloc(sizeof(oracle_path) * (size_t)(d->np + 1));
    int64_t XD, OD;
    int YD;
    if (build_paths(d, pt, &XD, &OD, &YD) != 0) {
        free(pt);
        return -1;
    }
    (void)N;
    (void)E;
    const int U = d->U, P = d->np;
#pragma omp parallel for schedule(dynamic, 4)
    for (int64_t k = 0; k < nrows; ++k) {
        int64_t r = rows ? rows[k] : k;
        double *o = out_rows + k * OD;
        for (int64_t j = 0; j < OD; ++j) o[j] = 0.0;
        for (int64_t e = rowptr[r]; e < rowptr[r + 1]; ++e) {
            int64_t s = src[e];
            for (int p = 0; p < P; ++p) {
                const oracle_path *q = &pt[p];
                for (int u = 0; u < U; ++u) {
                    double w = W[(e * P + p) * U + u];
                    for (int t = 0; t < q->nnz; ++t) {
                        double xv = x[s * XD + q->xoff + (int64_t)(u * q->xu) * q->n1 + q->m1[t]];
                        double yv = Y[e * YD + q->yoff + q->m2[t]];
                        o[q->ooff + (int64_t)(u * q->ou) * q->n3 + q->m3[t]] += q->c[t] * xv * yv * w;
                    }
                }
            }
        }
    }
    free(pt);
    return 0;
}

/* ------------------------------------------------------------------ */
/* Vector-Jacobian product.                                            */
/* For the loss <g, f(x, Y, W)>:                                        */
/*   gW[e,p,u]   = sum_t c x[s,u,m1] Y[e,m2] g[r,u,m3]                  */
/*   gY[e,l2 m2] = sum_{p with Y degree l2} sum_u sum_t c x[s,u,m1] W[e,p,u] g[r,u,m3] */
/*   gx[s,u,m1]  = sum_{e with src[e]=s} sum_p sum_t c Y[e,m2] W[e,p,u] g[r,u,m3]     */
/* ------------------------------------------------------------------ */

/* gW and gY for the listed edges (edges == NULL: all E edges in order).
 * gW_rows[k, P*U], gY_rows[k, YD]; either output pointer may be NULL. */
int oracle_bwd_edges(const oracle_desc *d, int64_t N, int64_t E,
                     const int32_t *rowptr, const int32_t *src, const double *x,
                     const double *Y, const double *W, const double *g,
                     const int64_t *edges, int64_t nedges, double *gW_rows,
                     double *gY_rows) {
    oracle_path *pt = (oracle_path *)malloc(sizeof(oracle_path) * (size_t)(d->np + 1));
    int64_t XD, OD;
    int YD;
    if (build_paths(d, pt, &XD, &OD, &YD) != 0) {
        free(pt);
        return -1;
    }
    int32_t *recv = (int32_t *)malloc(sizeof(int32_t) * (size_t)(E > 0 ? E : 1));
    edge_receivers(N, rowptr, recv);
    const int U = d->U, P = d->np;
#pragma omp parallel for schedule(dynamic, 16)
    for (int64_t k = 0; k < nedges; ++k) {
        int64_t e = edges ? edges[k] : k;
        int64_t s = src[e], r = recv[e];
        if (gW_rows) {
            for (int p = 0; p < P; ++p) {
                const oracle_path *q = &pt[p];
                for (int u = 0; u < U; ++u) {
                    double acc = 0.0;
                    for (int t = 0; t < q->nnz; ++t) {
                        double xv = x[s * XD + q->xoff + (int64_t)(u * q->xu) * q->n1 + q->m1[t]];
                        double yv = Y[e * YD + q->yoff + q->m2[t]];
                        double gv = g[r * OD + q->ooff + (int64_t)(u * q->ou) * q->n3 + q->m3[t]];
                        acc += q->c[t] * xv * yv * gv;
                    }
                    gW_rows[k * P * U + (int64_t)p * U + u] = acc;
                }
            }
        }
        if (gY_rows) {
            double *gy = gY_rows + k * YD;
            for (int j = 0; j < YD; ++j) gy[j] = 0.0;
            for (int p = 0; p < P; ++p) {
                const oracle_path *q = &pt[p];
                for (int u = 0; u < U; ++u) {
                    double w = W[(e * P + p) * U + u];
                    for (int t = 0; t < q->nnz; ++t) {
                        double xv = x[s * XD + q->xoff + (int64_t)(u * q->xu) * q->n1 + q->m1[t]];
                        double gv = g[r * OD + q->ooff + (int64_t)(u * q->ou) * q->n3 + q->m3[t]];
                        gy[q->yoff + q->m2[t]] += q->c[t] * xv * w * gv;
                    }
                }
            }
        }
    }
    free(recv);
    free(pt);
    return 0;
}

/* gx for the listed senders (senders == NULL: all N in order), gx_rows[k, XD].
 * Each sender sums its outgoing edges in increasing edge id. */
int oracle_bwd_gx(const oracle_desc *d, int64_t N, int64_t E, const int32_t *rowptr,
                  const int32_t *src, const double *Y, const double *W,
                  const double *g, const int64_t *senders, int64_t nsend,
                  double *gx_rows) {
    oracle_path *pt = (oracle_path *)malloc(sizeof(oracle_path) * (size_t)(d->np + 1));
    int64_t XD, OD;
    int YD;
    if (build_paths(d, pt, &XD, &OD, &YD) != 0) {
        free(pt);
        return -1;
    }
    int32_t *recv = (int32_t *)malloc(sizeof(int32_t) * (size_t)(E > 0 ? E : 1));
    int32_t *srowptr = (int32_t *)malloc(sizeof(int32_t) * (size_t)(N + 1));
    int32_t *sperm = (int32_t *)malloc(sizeof(int32_t) * (size_t)(E > 0 ? E : 1));
    edge_receivers(N, rowptr, recv);
    oracle_sender_csr(N, E, src, srowptr, sperm);
    const int U = d->U, P = d->np;
#pragma omp parallel for schedule(dynamic, 4)
    for (int64_t k = 0; k < nsend; ++k) {
        int64_t s = senders ? senders[k] : k;
        double *gx = gx_rows + k * XD;
        for (int64_t j = 0; j < XD; ++j) gx[j] = 0.0;
        for (int64_t j = srowptr[s]; j < srowptr[s + 1]; ++j) {
            int64_t e = sperm[j], r = recv[e];
            for (int p = 0; p < P; ++p) {
                const oracle_path *q = &pt[p];
                for (int u = 0; u < U; ++u) {
                    double w = W[(e * P + p) * U + u];
                    for (int t = 0; t < q->nnz; ++t) {
                        double yv = Y[e * YD + q->yoff + q->m2[t]];
                        double gv = g[r * OD + q->ooff + (int64_t)(u * q->ou) * q->n3 + q->m3[t]];
                        gx[q->xoff + (int64_t)(u * q->xu) * q->n1 + q->m1[t]] += q->c[t] * yv * w * gv;
                    }
                }
            }
        }
    }
    free(sperm);
    free(srowptr);
    free(recv);
    free(pt);
    return 0;
}

/* ------------------------------------------------------------------ */
/* Double backward.                                                     */
/* With f linear in each of x, Y, W and the VJP components              */
/*   gx = Bx(Y,W,g), gY = BY(x,W,g), gW = BW(x,Y,g),                    */
/* the scalar S = <ggx,gx> + <ggY,gY> + <ggW,gW> equals                 */
/*   <g, f(ggx,Y,W) + f(x,ggY,W) + f(x,Y,ggW)>,                         */
/* so its gradients are                                                 */
/*   dg = f(ggx,Y,W) + f(x,ggY,W) + f(x,Y,ggW)                          */
/*   dx = Bx(ggY,W,g) + Bx(Y,ggW,g)                                     */
/*   dY = BY(ggx,W,g) + BY(x,ggW,g)                                     */
/*   dW = BW(ggx,Y,g) + BW(x,ggY,g).                                    */
/* A NULL tangent is zero.                                              */
/* ------------------------------------------------------------------ */

static void axpy(double *y, const double *x, int64_t n) {
    for (int64_t i = 0; i < n; ++i) y[i] += x[i];
}

/* Outputs cover the listed rows (dg: receivers `rows`; dx: `senders`;
 * dY, dW: `edges`); a NULL list means all rows in order.  A NULL output is
 * not computed. */
int oracle_dbwd(const oracle_desc *d, int64_t N, int64_t E, const int32_t *rowptr,
                const int32_t *src, const double *x, const double *Y, const double *W,
                const double *g, const double *ggx, const double *ggY,
                const double *ggW, const int64_t *rows, int64_t nrows,
                const int64_t *edges, int64_t nedges, const int64_t *senders,
                int64_t nsend, double *dx, double *dY, double *dW, double *dg) {
    oracle_path *pt = (oracle_path *)malloc(sizeof(oracle_path) * (size_t)(d->np + 1));
    int64_t XD, OD;
    int YD;
    int rc = build_paths(d, pt, &XD, &OD, &YD);
    free(pt);
    if (rc != 0) return -1;
    const int64_t PU = (int64_t)d->np * d->U;
    if (dg) {
        double *to = (double *)malloc(sizeof(double) * (size_t)(nrows * OD + 1));
        memset(dg, 0, sizeof(double) * (size_t)(nrows * OD));
        if (ggx) { oracle_fwd(d, N, E, rowptr, src, ggx, Y, W, rows, nrows, to); axpy(dg, to, nrows * OD); }
        if (ggY) { oracle_fwd(d, N, E, rowptr, src, x, ggY, W, rows, nrows, to); axpy(dg, to, nrows * OD); }
        if (ggW) { oracle_fwd(d, N, E, rowptr, src, x, Y, ggW, rows, nrows, to); axpy(dg, to, nrows * OD); }
        free(to);
    }
    if (dx) {
        double *tx = (double *)malloc(sizeof(double) * (size_t)(nsend * XD + 1));
        memset(dx, 0, sizeof(double) * (size_t)(nsend * XD));
        if (ggY) { oracle_bwd_gx(d, N, E, rowptr, src, ggY, W, g, senders, nsend, tx); axpy(dx, tx, nsend * XD); }
        if (ggW) { oracle_bwd_gx(d, N, E, rowptr, src, Y, ggW, g, senders, nsend, tx); axpy(dx, tx, nsend * XD); }
        free(tx);
    }
    if (dY) {
        double *tY = (double *)malloc(sizeof(double) * (size_t)(nedges * YD + 1));
        memset(dY, 0, sizeof(double) * (size_t)(nedges * YD));
        if (ggx) { oracle_bwd_edges(d, N, E, rowptr, src, ggx, Y, W, g, edges, nedges, NULL, tY); axpy(dY, tY, nedges * YD); }
        if (ggW) { oracle_bwd_edges(d, N, E, rowptr, src, x, Y, ggW, g, edges, nedges, NULL, tY); axpy(dY, tY, nedges * YD); }
        free(tY);
    }
    if (dW) {
        double *tW = (double *)malloc(sizeof(double) * (size_t)(nedges * PU + 1));
        memset(dW, 0, sizeof(double) * (size_t)(nedges * PU));
        if (ggx) { oracle_bwd_edges(d, N, E, rowptr, src, ggx, Y, W, g, edges, nedges, tW, NULL); axpy(dW, tW, nedges * PU); }
        if (ggY) { oracle_bwd_edges(d, N, E, rowptr, src, x, ggY, W, g, edges, nedges, tW, NULL); axpy(dW, tW, nedges * PU); }
        free(tW);
    }
    return 0;
}

/* Number of OpenMP threads the oracle's parallel loops use. */
int oracle_num_threads(void) {
#ifdef _OPENMP
    extern int omp_get_max_threads(void);
    return omp_get_max_threads();
#else
    return 1;
#endif
}

/* Sets that number (for timing the oracle on one thread); results do not depend on it. */
void oracle_set_num_threads(int n) {
#ifdef _OPENMP
    extern void omp_set_num_threads(int);
    if (n > 0) omp_set_num_threads(n);
#else
    (void)n;
#endif
}
