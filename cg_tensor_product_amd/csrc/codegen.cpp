// HIP source emission for one plan.
//
// The sparse CG contraction of every path is unrolled into straight-line
// multiply-add code with the coefficients as literals, so each lane keeps its
// operands in registers and runs a long independent instruction stream (the
// register-resident sub-kernel idea of "An Efficient Sparse Kernel Generator for
// O(3)-Equivariant Deep Networks", abstract).  Nothing is gathered from a table
// at run time.
//
// Forward, per edge and lane (channel u), for every (x block i1, Y degree l2):
//   z[m1][m2] = x[m1] * Y[l2, m2]                    (shared by the paths of the pair)
//   t[m3]     = sum_{(m1,m2,m3) in nz(p)} c * z[m1][m2]
//   acc_p[m3] += W[p] * t[m3]
// Backward, per path p, with g the lane's output-gradient block of p:
//   T[m1][m2] = sum_{m3} c * g[m3]
//   q[m1]     = sum_{m2} Y[m2] T[m1][m2]   ->  gW[p] += sum_{m1} x[m1] q[m1]
//                                              gx[m1] += W[p] q[m1]
//   s[m2]     = sum_{m1} x[m1] T[m1][m2]   ->  gY[m2] += W[p] s[m2]
#include <cstdio>
#include <map>
#include <set>
#include <sstream>
#include <string>

#include "planner.hpp"

namespace oeq {

extern const char *kKernelTemplate;

namespace {

std::string lit(double v) {
    char buf[64];
    std::snprintf(buf, sizeof buf, "real_t(%.17g)", v);
    return buf;
}

// "acc = fma(c, v, acc)" with the trivial coefficients spelled out.
std::string fma_term(const std::string &acc, double c, const std::string &v, bool first) {
    if (first) {
        if (c == 1.0) return acc + " = " + v + ";";
        if (c == -1.0) return acc + " = -" + v + ";";
        return acc + " = " + lit(c) + " * " + v + ";";
    }
    if (c == 1.0) return acc + " += " + v + ";";
    if (c == -1.0) return acc + " -= " + v + ";";
    return acc + " = fmar(" + lit(c) + ", " + v + ", " + acc + ");";
}

void emit_moves(std::ostringstream &o, const oeq_plan &p) {
    // x row <-> registers
    o << "__device__ __forceinline__ void g_load_x(const real_t *__restrict__ xr, int u, real_t (&v)[NXC]) {\n";
    for (const auto &b : p.xb) {
        const int n = 2 * b.l + 1;
        o << "  { const real_t *q = xr + " << b.row_off << "LL + (i64)u * " << n << ";";
        for (int m = 0; m < n; ++m) o << " v[" << b.lane_off + m << "] = q[" << m << "];";
        o << " }\n";
    }
    o << "}\n";
    o << "__device__ __forceinline__ void g_store_x(real_t *__restrict__ xr, int u, const real_t (&v)[NXC]) {\n";
    for (const auto &b : p.xb) {
        const int n = 2 * b.l + 1;
        o << "  { real_t *q = xr + " << b.row_off << "LL + (i64)u * " << n << ";";
        for (int m = 0; m < n; ++m) o << " q[" << m << "] = v[" << b.lane_off + m << "];";
        o << " }\n";
    }
    o << "}\n";
    // x-gradient scatter: with XT the block is addressed m-major (element m*U + u),
    // so consecutive lanes hit consecutive addresses; oeq_x_untranspose restores
    // the u-major layout afterwards.
    o << "__device__ __forceinline__ void g_atomic_x(real_t *__restrict__ xr, int u, const real_t (&v)[NXC]) {\n";
    for (const auto &b : p.xb) {
        const int n = 2 * b.l + 1;
        if (p.xt) {
            o << "  { real_t *q = xr + " << b.row_off << "LL + u;";
            for (int m = 0; m < n; ++m)
                o << " atomicAdd(q + " << static_cast<int64_t>(m) * p.U << ", v[" << b.lane_off + m << "]);";
        } else {
            o << "  { real_t *q = xr + " << b.row_off << "LL + (i64)u * " << n << ";";
            for (int m = 0; m < n; ++m) o << " atomicAdd(q + " << m << ", v[" << b.lane_off + m << "]);";
        }
        o << " }\n";
    }
    o << "}\n";
    // m-major -> u-major inside one node row held in LDS
    o << "__device__ __forceinline__ void g_untranspose_row(const real_t *__restrict__ t, real_t *__restrict__ row) {\n";
    for (const auto &b : p.xb) {
        const int n = 2 * b.l + 1;
        o << "  for (int i = threadIdx.x; i < " << static_cast<int64_t>(n) * p.U << "; i += blockDim.x) { const int u = i / "
          << n << ", m = i - u * " << n << "; row[" << b.row_off << "LL + i] = t[" << b.row_off << "LL + m * " << p.U
          << " + u]; }\n";
    }
    o << "}\n";
    // output row <-> registers
    o << "__device__ __forceinline__ void g_load_g(const real_t *__restrict__ gr, int u, real_t (&v)[NOC]) {\n";
    for (const auto &b : p.ob) {
        const int n = 2 * b.l + 1;
        o << "  { const real_t *q = gr + " << b.row_off << "LL + (i64)u * " << n << ";";
        for (int m = 0; m < n; ++m) o << " v[" << b.lane_off + m << "] = q[" << m << "];";
        o << " }\n";
    }
    o << "}\n";
    o << "__device__ __forceinline__ void g_store_out(real_t *__restrict__ orow, int u, const real_t (&v)[NOC]) {\n";
    for (const auto &b : p.ob) {
        const int n = 2 * b.l + 1;
        o << "  { real_t *q = orow + " << b.row_off << "LL + (i64)u * " << n << ";";
        for (int m = 0; m < n; ++m) o << " q[" << m << "] = v[" << b.lane_off + m << "];";
        o << " }\n";
    }
    o << "}\n";
}

void emit_fwd_edge(std::ostringstream &o, const oeq_plan &p) {
    o << "__device__ __forceinline__ void g_fwd_edge(const real_t (&x)[NXC], const real_t (&y)[YD], "
         "const real_t (&w)[P], real_t (&acc)[NOC]) {\n";
    // group the paths by (x block, l2): the products x*Y are shared inside a group
    std::map<std::pair<int, int>, std::vector<int>> groups;
    for (size_t k = 0; k < p.paths.size(); ++k)
        groups[{p.paths[k].i1, p.paths[k].l2}].push_back(static_cast<int>(k));
    for (const auto &gkv : groups) {
        const int i1 = gkv.first.first, l2 = gkv.first.second;
        const auto &xb = p.xb[i1];
        std::set<std::pair<int, int>> used;
        for (int k : gkv.second)
            for (const auto &nz : p.paths[k].nz) used.insert({nz.m1, nz.m2});
        o << "  { // x block " << i1 << " (l=" << xb.l << ") x Y l=" << l2 << "\n";
        for (const auto &ab : used)
            o << "    const real_t z" << ab.first << "_" << ab.second << " = x[" << xb.lane_off + ab.first
              << "] * y[" << l2 * l2 + ab.second << "];\n";
        for (int k : gkv.second) {
            const Path &pa = p.paths[k];
            const auto &obk = p.ob[pa.ob];
            o << "    { // path " << k << ": " << pa.l1 << " x " << pa.l2 << " -> " << pa.l3 << "\n";
            for (int m3 = 0; m3 < 2 * pa.l3 + 1; ++m3) {
                bool first = true;
                std::ostringstream line;
                for (const auto &nz : pa.nz) {
                    if (nz.m3 != m3) continue;
                    line << " " << fma_term("t", nz.c,
                                            "z" + std::to_string(nz.m1) + "_" + std::to_string(nz.m2), first);
                    first = false;
                }
                if (first) continue;  // no coefficient reaches this m3
                const std::string a = "acc[" + std::to_string(obk.lane_off + m3) + "]";
                o << "      { real_t t;" << line.str() << " " << a << " = fmar(w[" << k << "], t, " << a
                  << "); }\n";
            }
            o << "    }\n";
        }
        o << "  }\n";
    }
    o << "}\n";
}

void emit_bwd_edge(std::ostringstream &o, const oeq_plan &p) {
    o << "template <bool GW, bool GY, bool GX>\n"
         "__device__ __forceinline__ void g_bwd_edge(const real_t (&x)[NXC], const real_t (&y)[YD], "
         "const real_t (&w)[P], const real_t (&g)[NOC], real_t (&gw)[P], real_t (&gy)[YD], real_t (&gx)[NXC]) {\n";
    for (size_t k = 0; k < p.paths.size(); ++k) {
        const Path &pa = p.paths[k];
        const auto &xb = p.xb[pa.i1];
        const auto &obk = p.ob[pa.ob];
        const int n1 = 2 * pa.l1 + 1, n2 = 2 * pa.l2 + 1;
        const int yo = pa.l2 * pa.l2;
        o << "  { // path " << k << ": " << pa.l1 << " x " << pa.l2 << " -> " << pa.l3 << "\n";
        // T[a][b] = sum_m3 c g[m3]
        std::map<std::pair<int, int>, std::vector<const NonZero *>> T;
        for (const auto &nz : pa.nz) T[{nz.m1, nz.m2}].push_back(&nz);
        for (const auto &tkv : T) {
            const std::string nm = "T" + std::to_string(tkv.first.first) + "_" + std::to_string(tkv.first.second);
            o << "    real_t " << nm << ";";
            bool first = true;
            for (const NonZero *nz : tkv.second) {
                o << " " << fma_term(nm, nz->c, "g[" + std::to_string(obk.lane_off + nz->m3) + "]", first);
                first = false;
            }
            o << "\n";
        }
        // q[a] = sum_b y[b] T[a][b]
        o << "    if constexpr (GW || GX) {\n";
        for (int a = 0; a < n1; ++a) {
            bool first = true;
            std::ostringstream line;
            for (const auto &tkv : T) {
                if (tkv.first.first != a) continue;
                const std::string tn = "T" + std::to_string(a) + "_" + std::to_string(tkv.first.second);
                const std::string yv = "y[" + std::to_string(yo + tkv.first.second) + "]";
                if (first)
                    line << " q = " << yv << " * " << tn << ";";
                else
                    line << " q = fmar(" << yv << ", " << tn << ", q);";
                first = false;
            }
            if (first) continue;
            o << "      { real_t q;" << line.str();
            o << " if constexpr (GW) gw[" << k << "] = fmar(x[" << xb.lane_off + a << "], q, gw[" << k
              << "]);";
            o << " if constexpr (GX) gx[" << xb.lane_off + a << "] = fmar(w[" << k << "], q, gx["
              << xb.lane_off + a << "]); }\n";
        }
        o << "    }\n";
        // s[b] = sum_a x[a] T[a][b]
        o << "    if constexpr (GY) {\n";
        for (int b = 0; b < n2; ++b) {
            bool first = true;
            std::ostringstream line;
            for (const auto &tkv : T) {
                if (tkv.first.second != b) continue;
                const std::string tn = "T" + std::to_string(tkv.first.first) + "_" + std::to_string(b);
                const std::string xv = "x[" + std::to_string(xb.lane_off + tkv.first.first) + "]";
                if (first)
                    line << " s = " << xv << " * " << tn << ";";
                else
                    line << " s = fmar(" << xv << ", " << tn << ", s);";
                first = false;
            }
            if (first) continue;
            o << "      { real_t s;" << line.str() << " gy[" << yo + b << "] = fmar(w[" << k
              << "], s, gy[" << yo + b << "]); }\n";
        }
        o << "    }\n";
        o << "  }\n";
    }
    o << "}\n";
}

}  // namespace

std::string emit_source(const oeq_plan &p) {
    std::ostringstream o;
    int py = 1, lgpy = 0;
    while (py < p.YD) {
        py <<= 1;
        ++lgpy;
    }
    o << "// Generated for: U=" << p.U << ", x blocks";
    for (const auto &b : p.xb) o << " " << b.l << (b.parity > 0 ? "e" : "o");
    o << ", Y degrees 0.." << p.L << ", " << p.paths.size() << " paths, " << p.total_nnz
      << " CG non-zeros, dtype " << (p.dtype == OEQ_F64 ? "f64" : "f32") << "\n";
    o << "typedef " << (p.dtype == OEQ_F64 ? "double" : "float") << " real_t;\n";
    o << "typedef long long i64;\n";
    o << "__device__ __forceinline__ float fmar(float a, float b, float c) { return __builtin_fmaf(a, b, c); }\n";
    o << "__device__ __forceinline__ double fmar(double a, double b, double c) { return __builtin_fma(a, b, c); }\n";
    o << "constexpr int U = " << p.U << ";\n";
    o << "constexpr int UCH = " << p.uch << ";\n";
    o << "constexpr int NXC = " << p.NXC << ";\n";
    o << "constexpr int NOC = " << p.NOC << ";\n";
    o << "constexpr int P = " << p.paths.size() << ";\n";
    o << "constexpr int YD = " << p.YD << ";\n";
    o << "constexpr int PY = " << py << ";\n";
    o << "constexpr int LGPY = " << lgpy << ";\n";
    o << "constexpr int GY_TILE = " << p.gy_tile << ";\n";
    o << "constexpr i64 XD = " << p.XD << "LL;\n";
    o << "constexpr i64 OD = " << p.OD << "LL;\n";
    o << "constexpr bool XT = " << (p.xt ? "true" : "false") << ";\n";
    emit_moves(o, p);
    emit_fwd_edge(o, p);
    emit_bwd_edge(o, p);
    o << kKernelTemplate;
    return o.str();
}

}  // namespace oeq
