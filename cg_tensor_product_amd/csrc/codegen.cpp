// HIP source emission for one plan.
//
// The sparse CG contraction of every path is unrolled into straight-line
// multiply-add code with the coefficients as literals, so each lane keeps its
// operands in registers and runs a long independent instruction stream (the
// register-resident sub-kernel idea of "An Efficient Sparse Kernel Generator for
// O(3)-Equivariant Deep Networks", abstract).  Nothing is gathered from a table
// at run time.
//
// The paths are split into groups; one wave computes one group for 64 channels
// of one receiver, so a wave holds only its group's accumulators, weights and
// gradients (fewer registers, more waves in flight).  Each group becomes a
// struct FG<k> (forward) or BG<k> (backward passes) with static member functions
// working on compact per-group register arrays:
//   NX / NW / NO      x values, paths (weights) and output values per lane
//   load_x, load_w, load_g, store_w, store_out, store_x, atomic_x
//   edge              forward of one edge into the accumulators
//   vjp<GW, GY, GX>   the three VJP components of one edge (accumulating)
//
// Forward, per edge and lane (channel u), for every (x block i1, Y degree l2):
//   z[m1][m2] = x[m1] * Y[l2, m2]                    (shared by the paths of the pair)
//   t[m3]     = sum_{(m1,m2,m3) in nz(p)} c * z[m1][m2]
//   acc_p[m3] += W[p] * t[m3]
// VJP, per path p, with g the lane's output-gradient block of p:
//   T[m1][m2] = sum_{m3} c * g[m3]
//   q[m1]     = sum_{m2} Y[m2] T[m1][m2]   ->  gW[p] += sum_{m1} x[m1] q[m1]
//                                              gx[m1] += W[p] q[m1]
//   s[m2]     = sum_{m1} x[m1] T[m1][m2]   ->  gY[m2] += W[p] s[m2]
#include <algorithm>
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

std::string S(long long v) { return std::to_string(v); }

// Local register layout of one group.
struct Local {
    std::vector<int> paths;                 // global path ids, ascending
    std::map<int, int> xoff;                // x block -> local lane offset
    std::map<int, int> ooff;                // output block -> local lane offset
    std::map<int, int> widx;                // global path -> local weight index
    int nx = 0, nw = 0, no = 0;
};

// first: the plan's first group, which also owns the output blocks that no path writes
// (it stores their zeros, so that every output element is written)
Local make_local(const oeq_plan &p, const std::vector<int> &paths, bool first = false) {
    Local L;
    L.paths = paths;
    std::sort(L.paths.begin(), L.paths.end());
    std::set<int> xs, os;
    for (int k : L.paths) {
        xs.insert(p.paths[k].i1);
        os.insert(p.paths[k].ob);
    }
    if (first) {
        std::vector<bool> fed(p.ob.size(), false);
        for (const Path &pa : p.paths) fed[pa.ob] = true;
        for (size_t o = 0; o < p.ob.size(); ++o)
            if (!fed[o]) os.insert(static_cast<int>(o));
    }
    for (int i : xs) {
        L.xoff[i] = L.nx;
        L.nx += 2 * p.xb[i].l + 1;
    }
    for (int o : os) {
        L.ooff[o] = L.no;
        L.no += 2 * p.ob[o].l + 1;
    }
    for (int k : L.paths) L.widx[k] = L.nw++;
    return L;
}

// How a row move addresses a node row:
//   kRowLoad      an input row (x, gg_x, grad_out): blocks at row_off; a one-channel
//                 block is read by every lane (broadcast)
//   kRowGradient  an x-gradient row: U channels in every block, at exp_off
//   kRowOut       an output row: blocks at row_off; one-channel blocks are left out
//                 (the forward sums their channels separately)
enum RowKind { kRowLoad, kRowGradient, kRowOut };

// Moves between a node row (u-major blocks) and a lane's compact registers.
void emit_row_move(std::ostringstream &o, const oeq_plan &p, const char *sig, const std::map<int, int> &blocks,
                   const std::vector<Block> &bl, RowKind kind, const char *ptr, bool add = false) {
    const bool load = kind == kRowLoad;
    o << "  static __device__ __forceinline__ void " << sig << " {\n";
    for (const auto &kv : blocks) {
        const Block &b = bl[kv.first];
        const int n = 2 * b.l + 1;
        const bool single = b.mul != p.U;  // one channel against U > 1
        if (kind == kRowOut && single) continue;
        const int64_t off = kind == kRowGradient ? b.exp_off : b.row_off;
        o << "    { " << (load ? "const " : "") << "real_t *q = " << ptr << " + " << off << "LL";
        if (!(load && single)) o << " + (i64)u * " << n;
        o << ";";
        for (int m = 0; m < n; ++m) {
            if (load)
                o << " v[" << kv.second + m << "] = q[" << m << "];";
            else
                o << " q[" << m << "] " << (add ? "+=" : "=") << " v[" << kv.second + m << "];";
        }
        o << " }\n";
    }
    o << "  }\n";
}

// All double-backward terms of one edge in one pass (TM: tangents present, 1 gg_x = tx,
// 2 gg_Y = ty, 4 gg_W = tw), sharing what the separate forward and VJP calls would each
// recompute:
//   d_grad_out[m3] += w * sum C (tx y + x ty) + tw * sum C x y
//   T[m1,m2] = sum_m3 C g[m3]  (once per path, not once per tangent)
//   d_W += tx . (T y) + x . (T ty);  d_x[m1] += w (T ty)[m1] + tw (T y)[m1]
//   d_Y[m2] += w (tx T)[m2] + tw (x T)[m2]
void emit_dbwd_edge(std::ostringstream &o, const oeq_plan &p, const Local &L) {
    o << "  template <int TM, bool GW, bool GY, bool GX>\n"
         "  static __device__ __forceinline__ void dbwd_edge(const real_t (&x)[NX], const real_t (&y)[YD], "
         "const real_t (&w)[NW], const real_t (&tx)[NX], const real_t (&ty)[YD], const real_t (&tw)[NW], "
         "const real_t (&g)[NO], bool want_dg, real_t (&dg)[NO], real_t (&dw)[NW], real_t (&dy)[YD], "
         "real_t (&dx)[NX]) {\n"
         "    constexpr bool HX = (TM & 1) != 0, HY = (TM & 2) != 0, HW = (TM & 4) != 0;\n"
         "    constexpr bool NQY = (HX && GW) || (HW && GX), NQT = HY && (GW || GX), NSX = HW && GY, NST = HX && GY;\n";
    // d_grad_out
    o << "    if (want_dg) {\n";
    std::map<std::pair<int, int>, std::vector<int>> pairs;  // (x block, Y block) -> paths
    for (int k : L.paths) pairs[{p.paths[k].i1, p.paths[k].iy}].push_back(k);
    for (const auto &gkv : pairs) {
        const int i1 = gkv.first.first, iy = gkv.first.second, yo0 = p.yb[iy].lane_off;
        const int xo = L.xoff.at(i1);
        std::set<std::pair<int, int>> used;
        for (int k : gkv.second)
            for (const auto &nz : p.paths[k].nz) used.insert({nz.m1, nz.m2});
        o << "      { // x block " << i1 << " x Y block " << iy << "\n";
        for (const auto &ab : used) {
            const std::string xa = "[" + S(xo + ab.first) + "]", yb = "[" + S(yo0 + ab.second) + "]";
            const std::string nm = S(ab.first) + "_" + S(ab.second);
            o << "        real_t z" << nm << ", u" << nm << ";";
            o << " if constexpr (HW) z" << nm << " = x" << xa << " * y" << yb << ";";
            o << " if constexpr (HX && HY) u" << nm << " = fmar(x" << xa << ", ty" << yb << ", tx" << xa << " * y" << yb
              << "); else if constexpr (HX) u" << nm << " = tx" << xa << " * y" << yb << "; else if constexpr (HY) u"
              << nm << " = x" << xa << " * ty" << yb << ";\n";
        }
        for (int k : gkv.second) {
            const Path &pa = p.paths[k];
            const int oo = L.ooff.at(pa.ob), wk = L.widx.at(k);
            o << "        { // path " << k << "\n";
            for (int m3 = 0; m3 < 2 * pa.l3 + 1; ++m3) {
                bool first = true;
                std::ostringstream l0, l1;
                for (const auto &nz : pa.nz) {
                    if (nz.m3 != m3) continue;
                    const std::string nm = S(nz.m1) + "_" + S(nz.m2);
                    l0 << " " << fma_term("s0", nz.c, "z" + nm, first);
                    l1 << " " << fma_term("s1", nz.c, "u" + nm, first);
                    first = false;
                }
                if (first) continue;
                const std::string d = "dg[" + S(oo + m3) + "]";
                o << "          if constexpr (HX || HY) { real_t s1;" << l1.str() << " " << d << " = fmar(w[" << wk
                  << "], s1, " << d << "); }";
                o << " if constexpr (HW) { real_t s0;" << l0.str() << " " << d << " = fmar(tw[" << wk << "], s0, " << d
                  << "); }\n";
            }
            o << "        }\n";
        }
        o << "      }\n";
    }
    o << "    }\n";
    // d_W, d_Y, d_x from T = C g
    o << "    if constexpr (GW || GY || GX) {\n";
    for (int k : L.paths) {
        const Path &pa = p.paths[k];
        const int xo = L.xoff.at(pa.i1), oo = L.ooff.at(pa.ob), wk = L.widx.at(k);
        const int n1 = 2 * pa.l1 + 1, n2 = 2 * pa.l2 + 1, yo = pa.yoff;
        o << "    { // path " << k << "\n";
        std::map<std::pair<int, int>, std::vector<const NonZero *>> T;
        for (const auto &nz : pa.nz) T[{nz.m1, nz.m2}].push_back(&nz);
        for (const auto &tkv : T) {
            const std::string nm = "T" + S(tkv.first.first) + "_" + S(tkv.first.second);
            o << "      real_t " << nm << ";";
            bool first = true;
            for (const NonZero *nz : tkv.second) {
                o << " " << fma_term(nm, nz->c, "g[" + S(oo + nz->m3) + "]", first);
                first = false;
            }
            o << "\n";
        }
        o << "      if constexpr (GW || GX) {\n";
        for (int a = 0; a < n1; ++a) {
            std::ostringstream qy, qt;
            bool first = true;
            for (const auto &tkv : T) {
                if (tkv.first.first != a) continue;
                const std::string tn = "T" + S(a) + "_" + S(tkv.first.second);
                const std::string yi = "[" + S(yo + tkv.first.second) + "]";
                if (first) {
                    qy << " qy = y" << yi << " * " << tn << ";";
                    qt << " qt = ty" << yi << " * " << tn << ";";
                } else {
                    qy << " qy = fmar(y" << yi << ", " << tn << ", qy);";
                    qt << " qt = fmar(ty" << yi << ", " << tn << ", qt);";
                }
                first = false;
            }
            if (first) continue;
            const std::string xa = "[" + S(xo + a) + "]";
            o << "        { real_t qy, qt; if constexpr (NQY) {" << qy.str() << " } if constexpr (NQT) {" << qt.str()
              << " }";
            o << " if constexpr (GW && HX) dw[" << wk << "] = fmar(tx" << xa << ", qy, dw[" << wk << "]);";
            o << " if constexpr (GW && HY) dw[" << wk << "] = fmar(x" << xa << ", qt, dw[" << wk << "]);";
            o << " if constexpr (GX && HY) dx" << xa << " = fmar(w[" << wk << "], qt, dx" << xa << ");";
            o << " if constexpr (GX && HW) dx" << xa << " = fmar(tw[" << wk << "], qy, dx" << xa << "); }\n";
        }
        o << "      }\n";
        o << "      if constexpr (GY) {\n";
        for (int b = 0; b < n2; ++b) {
            std::ostringstream sx, st;
            bool first = true;
            for (const auto &tkv : T) {
                if (tkv.first.second != b) continue;
                const std::string tn = "T" + S(tkv.first.first) + "_" + S(b);
                const std::string xi = "[" + S(xo + tkv.first.first) + "]";
                if (first) {
                    sx << " sx = x" << xi << " * " << tn << ";";
                    st << " st = tx" << xi << " * " << tn << ";";
                } else {
                    sx << " sx = fmar(x" << xi << ", " << tn << ", sx);";
                    st << " st = fmar(tx" << xi << ", " << tn << ", st);";
                }
                first = false;
            }
            if (first) continue;
            const std::string d = "dy[" + S(yo + b) + "]";
            o << "        { real_t sx, st; if constexpr (NSX) {" << sx.str() << " } if constexpr (NST) {" << st.str()
              << " }";
            o << " if constexpr (HX) " << d << " = fmar(w[" << wk << "], st, " << d << ");";
            o << " if constexpr (HW) " << d << " = fmar(tw[" << wk << "], sx, " << d << "); }\n";
        }
        o << "      }\n";
        o << "    }\n";
    }
    o << "    }\n";
    o << "  }\n";
}


// Y-contracted CG entries of one forward group: for every path and every (m1, m3) that a
// non-zero reaches, M[m1][m3] = sum_{m2} C[m1][m2][m3] Y[l2, m2].  M depends on the edge
// only (not on the channel), so it is built once per edge (one lane per edge) and read by
// every channel lane from LDS.
struct MEntry {
    int path, m1, m3;
    std::vector<std::pair<int, double>> terms;  // (index into the edge's Y row, coefficient)
};

std::vector<MEntry> m_entries(const oeq_plan &p, const Local &L) {
    std::vector<MEntry> out;
    for (int k : L.paths) {
        const Path &pa = p.paths[k];
        std::map<std::pair<int, int>, std::vector<std::pair<int, double>>> by;  // (m3, m1) -> terms
        for (const auto &nz : pa.nz) by[{nz.m3, nz.m1}].push_back({pa.yoff + nz.m2, nz.c});
        for (const auto &kv : by) out.push_back({k, kv.first.second, kv.first.first, kv.second});
    }
    return out;
}

// Row stride of the M rows in elements: whole 16-byte vectors, an odd number of them, so
// that lanes writing consecutive rows with 16-byte stores hit distinct banks.
int m_stride(const oeq_plan &p, int entries) {
    const int ve = p.dtype == OEQ_F64 ? 2 : 4;
    int nv = (std::max(entries, 1) + ve - 1) / ve;
    if (nv % 2 == 0) ++nv;
    return nv * ve;
}

int group_m_stride(const oeq_plan &p, const std::vector<int> &paths) {
    return m_stride(p, static_cast<int>(m_entries(p, make_local(p, paths)).size()));
}

void emit_m_functions(std::ostringstream &o, const oeq_plan &p, const Local &L, int moff) {
    const std::vector<MEntry> ents = m_entries(p, L);
    const int sm = m_stride(p, static_cast<int>(ents.size()));
    const int ve = p.dtype == OEQ_F64 ? 2 : 4;
    o << "  static constexpr int KM = " << ents.size() << ", SM = " << sm << ", MOFF = " << moff << ";\n";
    // one edge's M row from its Y row, written to LDS with 16-byte stores
    o << "  static __device__ __forceinline__ void make_m(const real_t (&y)[YD], real_t *__restrict__ row) {\n";
    o << "    real_t m[SM];\n";
    for (int j = 0; j < sm; ++j) {
        if (j < static_cast<int>(ents.size())) {
            bool first = true;
            o << "   ";
            for (const auto &t : ents[j].terms) {
                o << " " << fma_term("m[" + S(j) + "]", t.second, "y[" + S(t.first) + "]", first);
                first = false;
            }
            o << "\n";
        } else {
            o << "    m[" << j << "] = real_t(0);\n";
        }
        if (j % ve == ve - 1) {
            // store each vector once formed, with a scheduling fence after it (the kernel's
            // register peak is in the edge loop, not in this build of the rows)
            const int k = j / ve;
            o << "    { vec16_t v;";
            for (int i = 0; i < ve; ++i) o << " v[" << i << "] = m[" << ve * k + i << "];";
            o << " reinterpret_cast<vec16_t *>(row)[" << k << "] = v; } M_FENCE();\n";
        }
    }
    o << "  }\n";
    // forward of one edge from its M row (in LDS)
    o << "  static __device__ __forceinline__ void edge_m(const real_t (&x)[NX], const real_t *__restrict__ row, "
         "const real_t (&w)[NW], real_t (&acc)[NO]) {\n";
    // each 16-byte vector of the row is read just before its first entry is used, so the
    // row is never held in registers whole
    o << "    const vec16_t *__restrict__ mv = reinterpret_cast<const vec16_t *>(row);\n";
    int loaded = -1;
    auto need = [&](size_t i) {
        const int v = static_cast<int>(i) / ve;
        std::string r;
        while (loaded < v) {
            ++loaded;
            r += "    const vec16_t v" + S(loaded) + " = mv[" + S(loaded) + "];\n";
        }
        return r;
    };
    auto mref = [&](size_t i) { return "v" + S(static_cast<long long>(i) / ve) + "[" + S(static_cast<long long>(i) % ve) + "]"; };
    // paths as [begin, end) ranges of entries
    std::vector<std::pair<size_t, size_t>> ranges;
    for (size_t a = 0; a < ents.size();) {
        size_t b = a;
        while (b < ents.size() && ents[b].path == ents[a].path) ++b;
        ranges.push_back({a, b});
        a = b;
    }
    // the vectors a path needs, declared one path ahead of its arithmetic (declaring the
    // whole row first, or fencing the scheduler between paths, raised the medium config's
    // forward from 131 to 202-215 registers)
    auto load_for = [&](size_t r) {
        std::string out;
        if (r < ranges.size())
            for (size_t i = ranges[r].first; i < ranges[r].second; ++i) out += need(i);
        return out;
    };
    o << load_for(0) << load_for(1);
    for (size_t r = 0; r < ranges.size(); ++r) {
        const size_t j = ranges[r].first, j1 = ranges[r].second;
        const int k = ents[j].path;
        if (r > 0) o << load_for(r + 1);
        const Path &pa = p.paths[k];
        const int xo = L.xoff.at(pa.i1), oo = L.ooff.at(pa.ob), wk = L.widx.at(k);
        std::set<int> m1s, m3s;
        for (size_t i = j; i < j1; ++i) {
            m1s.insert(ents[i].m1);
            m3s.insert(ents[i].m3);
        }
        // vectors are declared at function scope (a path's entries can share a vector
        // with the next path's)
        if (m1s.size() < m3s.size()) {
            // weight applied to x first: acc[m3] += sum_m1 M[m1][m3] (w x[m1])
            o << "    // path " << k << ": " << pa.l1 << " x " << pa.l2 << " -> " << pa.l3 << " (weight on x)\n";
            for (int a : m1s) o << "    const real_t wx" << k << "_" << a << " = w[" << wk << "] * x[" << xo + a << "];\n";
            for (size_t i = j; i < j1; ++i) {
                const std::string d = "acc[" + S(oo + ents[i].m3) + "]";
                o << need(i) << "    " << d << " = fmar(" << mref(i) << ", wx" << k << "_" << ents[i].m1 << ", " << d
                  << ");\n";
            }
        } else {
            // t[m3] = sum_m1 M[m1][m3] x[m1];  acc[m3] += w t[m3]
            o << "    // path " << k << ": " << pa.l1 << " x " << pa.l2 << " -> " << pa.l3 << "\n";
            size_t i = j;
            while (i < j1) {
                const int m3 = ents[i].m3;
                std::string pre = need(i);
                std::string line = "    { real_t t = " + mref(i) + " * x[" + S(xo + ents[i].m1) + "];";
                ++i;
                while (i < j1 && ents[i].m3 == m3) {
                    pre += need(i);
                    line += " t = fmar(" + mref(i) + ", x[" + S(xo + ents[i].m1) + "], t);";
                    ++i;
                }
                const std::string d = "acc[" + S(oo + m3) + "]";
                o << pre << line << " " << d << " = fmar(w[" << wk << "], t, " << d << "); }\n";
            }
        }
    }
    o << "  }\n";
}

// Elements of the one-channel output blocks that a group writes.
int group_nsum(const oeq_plan &p, const std::vector<int> &paths, bool first) {
    int n = 0;
    for (const auto &kv : make_local(p, paths, first).ooff)
        if (p.ob[kv.first].mul != p.U) n += 2 * p.ob[kv.first].l + 1;
    return n;
}

// Hessian-vector product terms of one edge from its M row (in LDS), for the tangent v on
// x: per path and m3, t[m3] = sum_m1 M[m1][m3] v[m1] (the forward of v, shared by two
// outputs), then d_grad_out[m3] += w t[m3] and d_W += g[m3] t[m3].  The Y gradient needs
// the uncontracted tables and is formed by dbwd_edge.
void emit_hvp_m(std::ostringstream &o, const oeq_plan &p, const Local &L) {
    const std::vector<MEntry> ents = m_entries(p, L);
    const int ve = p.dtype == OEQ_F64 ? 2 : 4;
    o << "  static __device__ __forceinline__ void hvp_m(const real_t (&v)[NX], const real_t *__restrict__ row, "
         "const real_t (&w)[NW], const real_t (&g)[NO], real_t (&dg)[NO], real_t (&dw)[NW]) {\n";
    o << "    const vec16_t *__restrict__ mv = reinterpret_cast<const vec16_t *>(row);\n";
    int loaded = -1;
    auto need = [&](size_t i) {
        const int vi = static_cast<int>(i) / ve;
        std::string r;
        while (loaded < vi) {
            ++loaded;
            r += "    const vec16_t v" + S(loaded) + " = mv[" + S(loaded) + "];\n";
        }
        return r;
    };
    auto mref = [&](size_t i) { return "v" + S(static_cast<long long>(i) / ve) + "[" + S(static_cast<long long>(i) % ve) + "]"; };
    size_t i = 0;
    while (i < ents.size()) {
        const int k = ents[i].path, m3 = ents[i].m3;
        const Path &pa = p.paths[k];
        const int xo = L.xoff.at(pa.i1), oo = L.ooff.at(pa.ob), wk = L.widx.at(k);
        std::string pre = need(i);
        std::string line = "    { real_t t = " + mref(i) + " * v[" + S(xo + ents[i].m1) + "];";
        ++i;
        while (i < ents.size() && ents[i].path == k && ents[i].m3 == m3) {
            pre += need(i);
            line += " t = fmar(" + mref(i) + ", v[" + S(xo + ents[i].m1) + "], t);";
            ++i;
        }
        const std::string d = "dg[" + S(oo + m3) + "]";
        o << pre << line << " " << d << " = fmar(w[" << wk << "], t, " << d << "); dw[" << wk << "] = fmar(g["
          << oo + m3 << "], t, dw[" << wk << "]); }\n";
    }
    o << "  }\n";
}

void emit_group(std::ostringstream &o, const oeq_plan &p, const char *name, int g, const std::vector<int> &paths,
                int moff = 0, int soff = 0) {
    const Local L = make_local(p, paths, g == 0);
    o << "template <> struct " << name << "<" << g << "> {\n";
    o << "  static constexpr int NX = " << L.nx << ", NW = " << L.nw << ", NO = " << L.no << ";\n";
    emit_row_move(o, p, "load_x(const real_t *__restrict__ xr, int u, real_t (&v)[NX])", L.xoff, p.xb, kRowLoad, "xr");
    emit_row_move(o, p, "store_x(real_t *__restrict__ xr, int u, const real_t (&v)[NX])", L.xoff, p.xb, kRowGradient,
                  "xr");
    emit_row_move(o, p, "load_g(const real_t *__restrict__ gr, int u, real_t (&v)[NO])", L.ooff, p.ob, kRowLoad, "gr");
    emit_row_move(o, p, "store_out(real_t *__restrict__ orow, int u, const real_t (&v)[NO])", L.ooff, p.ob, kRowOut,
                  "orow");
    // accumulating variants (double backward split into one pass per tangent)
    emit_row_move(o, p, "add_x(real_t *__restrict__ xr, int u, const real_t (&v)[NX])", L.xoff, p.xb, kRowGradient, "xr",
                  true);
    emit_row_move(o, p, "add_out(real_t *__restrict__ orow, int u, const real_t (&v)[NO])", L.ooff, p.ob, kRowOut,
                  "orow", true);
    // output blocks of one channel: this group's elements of them (the forward sums them
    // over the channels), at SOFF in the plan's list of such elements
    {
        int nsum = 0;
        std::ostringstream pick;
        for (const auto &kv : L.ooff) {
            const Block &b = p.ob[kv.first];
            if (b.mul == p.U) continue;
            for (int m = 0; m < 2 * b.l + 1; ++m) pick << " s[" << nsum++ << "] = v[" << kv.second + m << "];";
        }
        o << "  static constexpr int NSUM = " << nsum << ", SOFF = " << soff << ";\n";
        o << "  static __device__ __forceinline__ void sum_pick(const real_t (&v)[NO], real_t (&s)[NSUM > 0 ? NSUM : 1]) {"
          << (nsum ? pick.str() : std::string(" s[0] = real_t(0);")) << " }\n";
        // offsets of those elements in an output row (kernels that own one group per workgroup)
        o << "  static __device__ __forceinline__ i64 sum_off_g(int j) {";
        if (nsum) {
            o << " switch (j) {";
            int j = 0;
            for (const auto &kv : L.ooff) {
                const Block &b = p.ob[kv.first];
                if (b.mul == p.U) continue;
                for (int m = 0; m < 2 * b.l + 1; ++m) o << " case " << j++ << ": return " << b.row_off + m << ";";
            }
            o << " }";
        }
        o << " return 0; }\n";
    }
    // x-gradient scatter: with XT the block is addressed m-major (element m*U + u),
    // so consecutive lanes hit consecutive words; oeq_x_untranspose restores the
    // u-major layout afterwards.
    o << "  static __device__ __forceinline__ void atomic_x(real_t *__restrict__ xr, int u, const real_t (&v)[NX]) {\n";
    for (const auto &kv : L.xoff) {
        const Block &b = p.xb[kv.first];
        const int n = 2 * b.l + 1;
        if (p.xt) {
            o << "    { real_t *q = xr + " << b.exp_off << "LL + u;";
            for (int m = 0; m < n; ++m)
                o << " atomicAdd(q + " << S(static_cast<long long>(m) * p.U) << ", v[" << kv.second + m << "]);";
        } else {
            o << "    { real_t *q = xr + " << b.exp_off << "LL + (i64)u * " << n << ";";
            for (int m = 0; m < n; ++m) o << " atomicAdd(q + " << m << ", v[" << kv.second + m << "]);";
        }
        o << " }\n";
    }
    o << "  }\n";
    // output scatter of the sender-stationary forward: always m-major inside each
    // output block (element m*U + u); oeq_out_untranspose restores the row layout
    o << "  static __device__ __forceinline__ void atomic_out(real_t *__restrict__ orow, int u, const real_t (&v)[NO]) {\n";
    for (const auto &kv : L.ooff) {
        const Block &b = p.ob[kv.first];
        const int n = 2 * b.l + 1;
        o << "    { real_t *q = orow + " << b.row_off << "LL + u;";
        for (int m = 0; m < n; ++m)
            o << " atomicAdd(q + " << S(static_cast<long long>(m) * p.U) << ", v[" << kv.second + m << "]);";
        o << " }\n";
    }
    o << "  }\n";
    // weights: we = W + e*P*U
    o << "  static __device__ __forceinline__ void load_w(const real_t *__restrict__ we, int u, real_t (&v)[NW]) {";
    for (int k : L.paths) o << " v[" << L.widx.at(k) << "] = LDW(we + " << S(static_cast<long long>(k) * p.U) << " + u);";
    o << " }\n";
    // a row [P, U] that every workgroup reads (the radial network's output matrix): cached loads
    o << "  static __device__ __forceinline__ void load_wrow(const real_t *__restrict__ row, int u, real_t (&v)[NW]) {";
    for (int k : L.paths) o << " v[" << L.widx.at(k) << "] = row[" << S(static_cast<long long>(k) * p.U) << " + u];";
    o << " }\n";
    o << "  static __device__ __forceinline__ void store_w(real_t *__restrict__ ge, int u, const real_t (&v)[NW]) {";
    for (int k : L.paths) o << " STW(ge + " << S(static_cast<long long>(k) * p.U) << " + u, v[" << L.widx.at(k) << "]);";
    o << " }\n";
    o << "  static __device__ __forceinline__ void add_w(real_t *__restrict__ ge, int u, const real_t (&v)[NW]) {";
    for (int k : L.paths) {
        const std::string a = "ge + " + S(static_cast<long long>(k) * p.U) + " + u";
        o << " STW(" << a << ", LDW(" << a << ") + v[" << L.widx.at(k) << "]);";
    }
    o << " }\n";

    // forward of one edge
    o << "  static __device__ __forceinline__ void edge(const real_t (&x)[NX], const real_t (&y)[YD], "
         "const real_t (&w)[NW], real_t (&acc)[NO]) {\n";
    std::map<std::pair<int, int>, std::vector<int>> pairs;  // (x block, Y block) -> paths
    for (int k : L.paths) pairs[{p.paths[k].i1, p.paths[k].iy}].push_back(k);
    for (const auto &gkv : pairs) {
        const int i1 = gkv.first.first, iy = gkv.first.second;
        const int xo = L.xoff.at(i1);
        std::set<std::pair<int, int>> used;
        for (int k : gkv.second)
            for (const auto &nz : p.paths[k].nz) used.insert({nz.m1, nz.m2});
        o << "    { // x block " << i1 << " (l=" << p.xb[i1].l << ") x Y block " << iy << " (l=" << p.yb[iy].l
          << ")\n";
        for (const auto &ab : used)
            o << "      const real_t z" << ab.first << "_" << ab.second << " = x[" << xo + ab.first << "] * y["
              << p.yb[iy].lane_off + ab.second << "];\n";
        for (int k : gkv.second) {
            const Path &pa = p.paths[k];
            const int oo = L.ooff.at(pa.ob);
            o << "      { // path " << k << ": " << pa.l1 << " x " << pa.l2 << " -> " << pa.l3 << "\n";
            for (int m3 = 0; m3 < 2 * pa.l3 + 1; ++m3) {
                bool first = true;
                std::ostringstream line;
                for (const auto &nz : pa.nz) {
                    if (nz.m3 != m3) continue;
                    line << " " << fma_term("t", nz.c, "z" + S(nz.m1) + "_" + S(nz.m2), first);
                    first = false;
                }
                if (first) continue;  // no coefficient reaches this m3
                const std::string a = "acc[" + S(oo + m3) + "]";
                o << "        { real_t t;" << line.str() << " " << a << " = fmar(w[" << L.widx.at(k) << "], t, " << a
                  << "); }\n";
            }
            o << "      }\n";
        }
        o << "    }\n";
    }
    o << "  }\n";

    // VJP of one edge
    o << "  template <bool GW, bool GY, bool GX>\n"
         "  static __device__ __forceinline__ void vjp(const real_t (&x)[NX], const real_t (&y)[YD], "
         "const real_t (&w)[NW], const real_t (&g)[NO], real_t (&gw)[NW], real_t (&gy)[YD], real_t (&gx)[NX]) {\n";
    for (int k : L.paths) {
        const Path &pa = p.paths[k];
        const int xo = L.xoff.at(pa.i1), oo = L.ooff.at(pa.ob), wk = L.widx.at(k);
        const int n1 = 2 * pa.l1 + 1, n2 = 2 * pa.l2 + 1;
        const int yo = pa.yoff;
        o << "    { // path " << k << ": " << pa.l1 << " x " << pa.l2 << " -> " << pa.l3 << "\n";
        std::map<std::pair<int, int>, std::vector<const NonZero *>> T;
        for (const auto &nz : pa.nz) T[{nz.m1, nz.m2}].push_back(&nz);
        for (const auto &tkv : T) {
            const std::string nm = "T" + S(tkv.first.first) + "_" + S(tkv.first.second);
            o << "      real_t " << nm << ";";
            bool first = true;
            for (const NonZero *nz : tkv.second) {
                o << " " << fma_term(nm, nz->c, "g[" + S(oo + nz->m3) + "]", first);
                first = false;
            }
            o << "\n";
        }
        o << "      if constexpr (GW || GX) {\n";
        for (int a = 0; a < n1; ++a) {
            bool first = true;
            std::ostringstream line;
            for (const auto &tkv : T) {
                if (tkv.first.first != a) continue;
                const std::string tn = "T" + S(a) + "_" + S(tkv.first.second);
                const std::string yv = "y[" + S(yo + tkv.first.second) + "]";
                if (first)
                    line << " q = " << yv << " * " << tn << ";";
                else
                    line << " q = fmar(" << yv << ", " << tn << ", q);";
                first = false;
            }
            if (first) continue;
            o << "        { real_t q;" << line.str();
            o << " if constexpr (GW) gw[" << wk << "] = fmar(x[" << xo + a << "], q, gw[" << wk << "]);";
            o << " if constexpr (GX) gx[" << xo + a << "] = fmar(w[" << wk << "], q, gx[" << xo + a << "]); }\n";
        }
        o << "      }\n";
        o << "      if constexpr (GY) {\n";
        for (int b = 0; b < n2; ++b) {
            bool first = true;
            std::ostringstream line;
            for (const auto &tkv : T) {
                if (tkv.first.second != b) continue;
                const std::string tn = "T" + S(tkv.first.first) + "_" + S(b);
                const std::string xv = "x[" + S(xo + tkv.first.first) + "]";
                if (first)
                    line << " s = " << xv << " * " << tn << ";";
                else
                    line << " s = fmar(" << xv << ", " << tn << ", s);";
                first = false;
            }
            if (first) continue;
            o << "        { real_t s;" << line.str() << " gy[" << yo + b << "] = fmar(w[" << wk << "], s, gy[" << yo + b
              << "]); }\n";
        }
        o << "      }\n";
        o << "    }\n";
    }
    o << "  }\n";
    if (std::string(name) == "BG" || std::string(name) == "DG") emit_dbwd_edge(o, p, L);
    if (std::string(name) == "FG" && p.fwd_lds) emit_m_functions(o, p, L, moff);
    if (std::string(name) == "BG" && p.hvp_lds) {
        emit_m_functions(o, p, L, 0);
        emit_hvp_m(o, p, L);
    }
    o << "};\n";
}

void emit_untranspose(std::ostringstream &o, const oeq_plan &p) {
    // m-major -> u-major inside one node row held in LDS
    o << "__device__ __forceinline__ void g_untranspose_row(const real_t *__restrict__ t, real_t *__restrict__ row) {\n";
    for (const auto &b : p.xb) {
        const int n = 2 * b.l + 1;
        o << "  for (int i = threadIdx.x; i < " << S(static_cast<long long>(n) * p.U)
          << "; i += blockDim.x) { const int u = i / " << n << ", m = i - u * " << n << "; row[" << b.exp_off
          << "LL + i] = t[" << b.exp_off << "LL + m * " << p.U << " + u]; }\n";
    }
    o << "}\n";
    // the same for an output row, one block at a time through a buffer of the largest block
    int64_t big = 1;
    for (const auto &b : p.ob) big = std::max<int64_t>(big, static_cast<int64_t>(2 * b.l + 1) * p.U);
    o << "constexpr int OUT_BLOCK_MAX = " << big << ";\n";
    o << "__device__ __forceinline__ void g_untranspose_out_row(real_t *__restrict__ t, real_t *__restrict__ row) {\n";
    for (const auto &b : p.ob) {
        const int n = 2 * b.l + 1;
        const long long cnt = static_cast<long long>(n) * p.U;
        o << "  for (int i = threadIdx.x; i < " << cnt << "; i += blockDim.x) t[i] = row[" << b.row_off << "LL + i];\n";
        o << "  __syncthreads();\n";
        o << "  for (int i = threadIdx.x; i < " << cnt << "; i += blockDim.x) { const int u = i / " << n
          << ", m = i - u * " << n << "; row[" << b.row_off << "LL + i] = t[m * " << p.U << " + u]; }\n";
        o << "  __syncthreads();\n";
    }
    o << "}\n";
}

// Element c of a node's x-gradient row from its row with U channels in every block: a
// one-channel block's element is the sum of its U channel copies, added in channel order.
void emit_fold_x(std::ostringstream &o, const oeq_plan &p) {
    o << "__device__ __forceinline__ real_t fold_x_elem(const real_t *__restrict__ re, int c) {\n";
    for (const auto &b : p.xb) {
        const int n = 2 * b.l + 1;
        const int64_t end = b.row_off + static_cast<int64_t>(b.mul) * n;
        if (b.mul == p.U) {
            o << "  if (c < " << end << ") return re[c + " << b.exp_off - b.row_off << "LL];\n";
        } else {
            o << "  if (c < " << end << ") { const int m = c - " << b.row_off << "; real_t s = re[" << b.exp_off
              << "LL + m]; for (int u = 1; u < U; ++u) s += re[" << b.exp_off << "LL + (i64)u * " << n
              << " + m]; return s; }\n";
        }
    }
    o << "  return real_t(0);\n}\n";
}

}  // namespace

int hvp_m_elems(const oeq_plan &p) {
    int n = 0;
    for (size_t g = 0; g < p.bwd_groups.size(); ++g) n = std::max(n, group_m_stride(p, p.bwd_groups[g]));
    return n;
}

int fwd_m_elems(const oeq_plan &p) {
    int n = 0;
    for (const auto &g : p.fwd_groups) n += group_m_stride(p, g);
    return n;
}

std::string emit_source(const oeq_plan &p) {
    std::ostringstream o;
    int py = 1, lgpy = 0;
    while (py < p.YD) {
        py <<= 1;
        ++lgpy;
    }
    o << "// Generated for: U=" << p.U << ", x blocks";
    for (const auto &b : p.xb) o << " " << b.l << (b.parity > 0 ? "e" : "o");
    o << ", Y blocks";
    for (const auto &b : p.yb) o << " " << b.l << (b.parity > 0 ? "e" : "o");
    o << ", " << p.paths.size() << " paths, " << p.total_nnz
      << " CG non-zeros, dtype " << (p.dtype == OEQ_F64 ? "f64" : "f32") << "; forward groups of";
    for (const auto &g : p.fwd_groups) o << " " << g.size();
    o << " paths, backward groups of";
    for (const auto &g : p.bwd_groups) o << " " << g.size();
    o << ", double-backward groups of";
    for (const auto &g : p.dbwd_groups) o << " " << g.size();
    o << ", radial backward groups of";
    for (const auto &g : p.rad_groups) o << " " << g.size();
    o << " paths\n";
    o << "typedef " << (p.dtype == OEQ_F64 ? "double" : "float") << " real_t;\n";
    o << "typedef long long i64;\n";
    o << "__device__ __forceinline__ float fmar(float a, float b, float c) { return __builtin_fmaf(a, b, c); }\n";
    o << "__device__ __forceinline__ double fmar(double a, double b, double c) { return __builtin_fma(a, b, c); }\n";
    if (p.nt_w) {
        // W and its gradients are streamed once: non-temporal accesses keep them out of the way of x and g
        o << "#define LDW(ptr) __builtin_nontemporal_load(ptr)\n";
        o << "#define STW(ptr, v) __builtin_nontemporal_store((v), (ptr))\n";
    } else {
        o << "#define LDW(ptr) (*(ptr))\n";
        o << "#define STW(ptr, v) (*(ptr) = (v))\n";
    }
    // a scheduling barrier after the next edge's loads keeps them from being sunk
    // toward their uses, which would expose the full memory latency every edge
    o << (p.pin_fwd ? "#define PIN_FWD() __builtin_amdgcn_sched_barrier(0)\n" : "#define PIN_FWD() ((void)0)\n");
    o << (p.pin_bwd ? "#define PIN_BWD() __builtin_amdgcn_sched_barrier(0)\n" : "#define PIN_BWD() ((void)0)\n");
    // occupancy window handed to the compiler's scheduler (waves per SIMD)
    auto occ = [](const std::pair<int, int> &w) {
        return w.first > 0 ? "__attribute__((amdgpu_waves_per_eu(" + S(w.first) + ", " + S(w.second) + ")))"
                           : std::string();
    };
    o << "#define FWD_OCCUPANCY " << occ(p.fwd_waves) << "\n";
    o << "#define BWD_OCCUPANCY " << occ(p.bwd_waves) << "\n";
    o << "constexpr int U = " << p.U << ";\n";
    o << "constexpr int UCH = " << p.uch << ";\n";
    o << "constexpr int NGF = " << p.fwd_groups.size() << ";\n";
    o << "constexpr int NGB = " << p.bwd_groups.size() << ";\n";
    o << "constexpr int NGD = " << p.dbwd_groups.size() << ";\n";
    o << "constexpr bool DBWD_TWO_SETS = " << (p.dbwd_groups != p.bwd_groups ? "true" : "false") << ";\n";
    o << "constexpr int P = " << p.paths.size() << ";\n";
    o << "constexpr int LY = " << p.L << ";\n";
    o << "constexpr int YD = " << p.YD << ";\n";
    // element k of a Y row is element YSEL[k] of the harmonics of degrees 0..LY (the
    // forward and VJP from edge vectors evaluate those and keep the plan's blocks)
    o << "constexpr int YSEL[YD] = {";
    {
        bool first = true;
        for (const auto &b : p.yb)
            for (int m = 0; m < 2 * b.l + 1; ++m) {
                o << (first ? "" : ", ") << b.l * b.l + m;
                first = false;
            }
    }
    o << "};\n";
    o << "constexpr int PY = " << py << ";\n";
    o << "constexpr int LGPY = " << lgpy << ";\n";
    o << "constexpr int GY_TILE = " << p.gy_tile << ";\n";
    o << "constexpr i64 XD = " << p.XD << "LL;\n";
    o << "constexpr i64 OD = " << p.OD << "LL;\n";
    // x-gradient rows carry U channels in every block (GXD > XD with one-channel x blocks)
    o << "constexpr i64 GXD = " << p.GXD << "LL;\n";
    o << "constexpr bool XT = " << (p.xt ? "true" : "false") << ";\n";
    o << "template <int G> struct FG;\n";
    o << "template <int G> struct BG;\n";
    o << "template <int G> struct RG;\n";
    o << "template <int G> struct DG;\n";
    o << "constexpr int NGR = " << p.rad_groups.size() << ";\n";
    o << "constexpr bool FWD_LDS = " << (p.fwd_lds ? "true" : "false") << ";\n";
    o << "constexpr bool FWD_XCD = " << (p.fwd_xcd ? "true" : "false") << ";\n";
    o << "#define M_FENCE() __builtin_amdgcn_sched_barrier(0)\n";
    o << "constexpr int FWD_MT = " << p.fwd_tile << ";\n";
    o << "constexpr int FWD_PF = " << p.fwd_pf << ";\n";
    o << "constexpr int BWD_PF = " << p.bwd_pf << ";\n";
    // HVP from Y-contracted CG rows: tiles of HVP_MT edges, rows of at most HVP_M_MAX values
    o << "constexpr bool HVP_LDS = " << (p.hvp_lds ? "true" : "false") << ";\n";
    o << "constexpr int HVP_MT = " << p.hvp_tile << ";\n";
    o << "constexpr int HVP_M_MAX = " << (p.hvp_lds ? hvp_m_elems(p) : 0) << ";\n";
    o << "typedef real_t vec16_t __attribute__((ext_vector_type(" << (p.dtype == OEQ_F64 ? 2 : 4) << ")));\n";
    {
        int moff = 0, soff = 0;
        for (size_t g = 0; g < p.fwd_groups.size(); ++g) {
            emit_group(o, p, "FG", static_cast<int>(g), p.fwd_groups[g], moff, soff);
            moff += group_m_stride(p, p.fwd_groups[g]);
            soff += group_nsum(p, p.fwd_groups[g], g == 0);
        }
        // elements of one edge's M rows over all forward groups
        o << "constexpr int FWD_M_ELEMS = " << (p.fwd_lds ? moff : 0) << ";\n";
        // elements of the one-channel output blocks (in forward-group order) and their
        // offsets in an output row
        o << "constexpr int NSUMT = " << soff << ";\n";
        o << "__device__ __forceinline__ i64 sum_off(int t) {";
        if (soff > 0) {
            o << " switch (t) {";
            int t = 0;
            for (size_t g = 0; g < p.fwd_groups.size(); ++g) {
                for (const auto &kv : make_local(p, p.fwd_groups[g], g == 0).ooff) {
                    const Block &b = p.ob[kv.first];
                    if (b.mul == p.U) continue;
                    for (int m = 0; m < 2 * b.l + 1; ++m) o << " case " << t++ << ": return " << b.row_off + m << ";";
                }
            }
            o << " }";
        }
        o << " return 0; }\n";
    }
    for (size_t g = 0; g < p.bwd_groups.size(); ++g) emit_group(o, p, "BG", static_cast<int>(g), p.bwd_groups[g]);
    for (size_t g = 0; g < p.rad_groups.size(); ++g) emit_group(o, p, "RG", static_cast<int>(g), p.rad_groups[g]);
    if (p.dbwd_groups == p.bwd_groups) {
        o << "template <int G> struct DG : BG<G> {};\n";
    } else {
        for (size_t g = 0; g < p.dbwd_groups.size(); ++g)
            emit_group(o, p, "DG", static_cast<int>(g), p.dbwd_groups[g]);
    }
    {
        // one-channel output elements of the largest backward or double-backward group (the
        // double backward sums their d_grad_out over the channels in LDS)
        int mx = 0;
        for (size_t g = 0; g < p.bwd_groups.size(); ++g) mx = std::max(mx, group_nsum(p, p.bwd_groups[g], g == 0));
        for (size_t g = 0; g < p.dbwd_groups.size(); ++g) mx = std::max(mx, group_nsum(p, p.dbwd_groups[g], g == 0));
        o << "constexpr int DBWD_NSUM_MAX = " << mx << ";\n";
    }
    emit_untranspose(o, p);
    emit_fold_x(o, p);
    o << kKernelTemplate;
    return o.str();
}

}  // namespace oeq
