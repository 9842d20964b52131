// Path planning: descriptor validation, path enumeration, sparse CG tables and
// row layouts.
//
// A path couples x block i1 (degree l1, parity p1) with the Y harmonics of
// degree l2 into an output of degree l3; with no explicit list, every l3 allowed
// by the triangle rule |l1-l2| <= l3 <= l1+l2 (and l3 <= lmax_out) is used, with
// output parity p1 (-1)^l2, x blocks in descriptor order, then l2 ascending, then
// l3 ascending.  Each path keeps only the non-zero entries of its real-basis CG
// table (compact storage of the structurally non-zero part, as the UMA kernel
// work compacts its rotation blocks in "Optimize UMA SO2 and Wigner inference
// kernels").
#include <algorithm>
#include <cstdio>
#include <cstdlib>
#include <cstring>
#include <map>
#include <set>
#include <sstream>

#include "planner.hpp"

namespace oeq {

namespace {

oeq_status fail(std::string *why, oeq_status st, const std::string &msg) {
    if (why) *why = msg;
    return st;
}

}  // namespace

// Splits the paths into at most `want` groups by longest-processing-time
// assignment of indivisible units.  Paths that share an output block always
// stay together (a block is written by one wave); so do paths that share the
// (x block, l2) pair in the forward (they share products x*Y), and paths that
// share an x block in the backward passes (that block's gradient is then owned
// by one wave, so per-edge x-gradient rows never overlap).
std::vector<std::vector<int>> partition_paths(const oeq_plan &p, bool fwd, int want) {
    const int n = static_cast<int>(p.paths.size());
    std::vector<int> parent(n);
    for (int i = 0; i < n; ++i) parent[i] = i;
    auto find = [&](int a) {
        while (parent[a] != a) a = parent[a] = parent[parent[a]];
        return a;
    };
    auto unite = [&](int a, int b) { parent[find(a)] = find(b); };
    for (int a = 0; a < n; ++a)
        for (int b = a + 1; b < n; ++b) {
            const Path &pa = p.paths[a], &pb = p.paths[b];
            const bool same = fwd ? (pa.i1 == pb.i1 && pa.iy == pb.iy) : (pa.i1 == pb.i1);
            if (same || pa.ob == pb.ob) unite(a, b);
        }
    std::map<int, std::vector<int>> units;
    for (int k = 0; k < n; ++k) units[find(k)].push_back(k);
    std::vector<std::pair<double, std::vector<int>>> uc;
    for (auto &kv : units) {
        double c = 0.0;
        for (int k : kv.second) {
            const Path &pa = p.paths[k];
            const double nnz = static_cast<double>(pa.nz.size());
            c += fwd ? nnz + (2 * pa.l3 + 1) + (2 * pa.l1 + 1)
                     : nnz + 2.0 * (2 * pa.l1 + 1) * (2 * pa.l2 + 1) + 2 * (2 * pa.l1 + 1) + (2 * pa.l2 + 1);
        }
        uc.push_back({c, kv.second});
    }
    std::stable_sort(uc.begin(), uc.end(), [](const auto &a, const auto &b) { return a.first > b.first; });
    const int g = std::max(1, std::min(want, static_cast<int>(uc.size())));
    std::vector<std::vector<int>> groups(g);
    std::vector<double> load(g, 0.0);
    for (auto &u : uc) {
        const int t = static_cast<int>(std::min_element(load.begin(), load.end()) - load.begin());
        load[t] += u.first;
        groups[t].insert(groups[t].end(), u.second.begin(), u.second.end());
    }
    for (auto &gr : groups) std::sort(gr.begin(), gr.end());
    std::sort(groups.begin(), groups.end());
    return groups;
}

// Rough per-lane register demand of a group (values held across the edge loop
// plus the largest transient product set), used to choose the group count.
int group_registers(const oeq_plan &p, const std::vector<int> &paths, bool fwd) {
    std::set<int> xs, os;
    int transient = 0;
    for (int k : paths) {
        const Path &pa = p.paths[k];
        xs.insert(pa.i1);
        os.insert(pa.ob);
        transient = std::max(transient, (2 * pa.l1 + 1) * (2 * pa.l2 + 1));
    }
    int nx = 0, no = 0;
    for (int i : xs) nx += 2 * p.xb[i].l + 1;
    for (int o : os) no += 2 * p.ob[o].l + 1;
    const int nw = static_cast<int>(paths.size());
    const int vals = fwd ? no + 2 * (nx + nw) + transient : no + 2 * (nx + nw) + p.YD + nx + transient;
    return vals * (p.dtype == OEQ_F64 ? 2 : 1) + 20;
}

// The double backward's groups: as many as the indivisible units allow (at most 16 waves
// per workgroup). Measured with all three tangents (ms, 1 / 2 / 3 groups): large 6.78 / 5.15 /
// 4.81, wide 14.84 / 10.50 / 9.68, medium fp64 5.91 / 4.99 (two units); the medium fp32 plan
// runs its fused kernel on the backward groups (one group, no spill), so its split here is
// not used.
std::vector<std::vector<int>> choose_dbwd_groups(const oeq_plan &p) {
    const int max_g = std::max(1, 16 / p.uch);
    if (const char *e = std::getenv("OEQ_DBWD_GROUPS"))
        return partition_paths(p, false, std::max(1, std::min(std::atoi(e), max_g)));
    return partition_paths(p, false, max_g);
}

std::vector<std::vector<int>> choose_groups(const oeq_plan &p, bool fwd) {
    const char *env = std::getenv(fwd ? "OEQ_FWD_GROUPS" : "OEQ_BWD_GROUPS");
    const int max_g = std::max(1, 16 / p.uch);  // at most 16 waves per workgroup
    if (env) return partition_paths(p, fwd, std::max(1, std::min(std::atoi(env), max_g)));
    // Measured on MI355X: splitting the backward passes costs more (a lane
    // reduction of the Y-gradient per group and per edge) than the occupancy it
    // buys; the forward gains once one group would need more than ~160 registers.
    if (!fwd) return partition_paths(p, fwd, 1);
    const int budget = 160;
    std::vector<std::vector<int>> best = partition_paths(p, fwd, 1);
    for (int g = 1; g <= max_g; ++g) {
        auto cand = partition_paths(p, fwd, g);
        best = cand;
        int worst = 0;
        for (const auto &gr : cand) worst = std::max(worst, group_registers(p, gr, fwd));
        if (worst <= budget || static_cast<int>(cand.size()) < g) break;
    }
    return best;
}

oeq_status plan_build(const oeq_tp_desc *d, oeq_plan *p, std::string *why) {
    if (!d) return fail(why, OEQ_ERR_INVALID_ARG, "descriptor is NULL");
    if (d->dtype != OEQ_F32 && d->dtype != OEQ_F64)
        return fail(why, OEQ_ERR_UNSUPPORTED, "dtype must be OEQ_F32 or OEQ_F64");
    if (!d->x_irreps || d->n_x <= 0 || d->n_x > 16)
        return fail(why, OEQ_ERR_INVALID_ARG, "x_irreps must hold 1..16 blocks");
    p->dtype = d->dtype;
    // Y blocks: the given irreps, or the spherical harmonics 0..y_lmax (parity (-1)^l)
    if (d->y_irreps) {
        if (d->n_y <= 0 || d->n_y > 16) return fail(why, OEQ_ERR_INVALID_ARG, "y_irreps must hold 1..16 blocks");
        int off = 0;
        for (int j = 0; j < d->n_y; ++j) {
            const oeq_irrep &ir = d->y_irreps[j];
            if (ir.mul != 1) return fail(why, OEQ_ERR_UNSUPPORTED, "Y blocks must have multiplicity 1");
            if (ir.l < 0 || ir.l > kLMax) return fail(why, OEQ_ERR_UNSUPPORTED, "Y degree must be in 0..3");
            if (ir.parity != 1 && ir.parity != -1) return fail(why, OEQ_ERR_INVALID_ARG, "parity must be +1 or -1");
            p->yb.push_back({ir.l, ir.parity, off, off});
            off += 2 * ir.l + 1;
        }
    } else {
        if (d->y_lmax < 0 || d->y_lmax > kLMax) return fail(why, OEQ_ERR_UNSUPPORTED, "y_lmax must be in 0..3");
        for (int l = 0; l <= d->y_lmax; ++l) p->yb.push_back({l, (l % 2) ? -1 : 1, l * l, l * l});
    }
    p->YD = 0;
    p->L = 0;
    for (const Block &b : p->yb) {
        p->YD += 2 * b.l + 1;
        p->L = std::max(p->L, b.l);
        if (b.parity != ((b.l % 2) ? -1 : 1)) p->y_natural = false;
    }
    // the lane reduction of the Y gradient handles rows of up to 16 values
    if (p->YD > 16) return fail(why, OEQ_ERR_UNSUPPORTED, "Y rows wider than 16 values");
    // U: the largest x multiplicity.  A block of one channel (x or output) reduces a UVW
    // product to the channel-wise one: an x block broadcast against the U channels, an
    // output block that receives their sum.
    p->U = 0;
    for (int i = 0; i < d->n_x; ++i) {
        if (d->x_irreps[i].mul <= 0) return fail(why, OEQ_ERR_INVALID_ARG, "multiplicity must be >= 1");
        p->U = std::max(p->U, d->x_irreps[i].mul);
    }
    if (p->U > 1024) return fail(why, OEQ_ERR_UNSUPPORTED, "multiplicity above 1024");
    int lane = 0;
    int64_t row = 0;
    for (int i = 0; i < d->n_x; ++i) {
        const oeq_irrep &ir = d->x_irreps[i];
        if (ir.mul != p->U && ir.mul != 1)
            return fail(why, OEQ_ERR_UNSUPPORTED,
                        "x blocks must have U channels (the largest multiplicity) or one (broadcast)");
        if (ir.l < 0 || ir.l > kLMax) return fail(why, OEQ_ERR_UNSUPPORTED, "x degree must be in 0..3");
        if (ir.parity != 1 && ir.parity != -1) return fail(why, OEQ_ERR_INVALID_ARG, "parity must be +1 or -1");
        p->xb.push_back({ir.l, ir.parity, lane, row, ir.mul, static_cast<int64_t>(p->U) * lane});
        if (ir.mul != p->U) p->bcast_x = true;
        lane += 2 * ir.l + 1;
        row += static_cast<int64_t>(ir.mul) * (2 * ir.l + 1);
    }
    p->NXC = lane;
    p->XD = row;
    p->GXD = static_cast<int64_t>(p->U) * lane;

    // Output blocks and the path list.
    struct Raw { int i1, iy, ob; };
    std::vector<Raw> raw;
    std::vector<std::pair<int, int>> out_lp;  // (l, parity) of each output block
    std::vector<int> out_mul;                 // channels of each given output block
    if (d->paths == nullptr) {
        if (d->lmax_out < 0 || d->lmax_out > kLMax)
            return fail(why, OEQ_ERR_UNSUPPORTED, "lmax_out must be in 0..3");
        if (d->out_irreps) {
            if (d->n_out <= 0) return fail(why, OEQ_ERR_INVALID_ARG, "n_out must be positive");
            for (int o = 0; o < d->n_out; ++o) {
                const oeq_irrep &ir = d->out_irreps[o];
                if (ir.mul != p->U && ir.mul != 1)
                    return fail(why, OEQ_ERR_UNSUPPORTED, "output blocks must have U channels or one (a channel sum)");
                if (ir.l < 0 || ir.l > kLMax) return fail(why, OEQ_ERR_UNSUPPORTED, "output degree must be in 0..3");
                if (ir.parity != 1 && ir.parity != -1)
                    return fail(why, OEQ_ERR_INVALID_ARG, "parity must be +1 or -1");
                out_lp.push_back({ir.l, ir.parity});
                out_mul.push_back(ir.mul);
            }
        }
        for (int i = 0; i < d->n_x; ++i) {
            const int l1 = d->x_irreps[i].l, p1 = d->x_irreps[i].parity;
            for (int j = 0; j < static_cast<int>(p->yb.size()); ++j) {
                const int l2 = p->yb[j].l;
                const int p3 = p1 * p->yb[j].parity;
                const int hi = std::min(l1 + l2, static_cast<int>(d->lmax_out));
                for (int l3 = std::abs(l1 - l2); l3 <= hi; ++l3) {
                    if (d->out_irreps) {
                        // paths into a given output irrep are summed into its block
                        int ob = -1;
                        for (size_t o = 0; o < out_lp.size(); ++o)
                            if (out_lp[o].first == l3 && out_lp[o].second == p3) {
                                ob = static_cast<int>(o);
                                break;
                            }
                        if (ob >= 0) raw.push_back({i, j, ob});
                    } else {
                        raw.push_back({i, j, static_cast<int>(out_lp.size())});
                        out_lp.push_back({l3, p3});
                        out_mul.push_back(p->U);
                    }
                }
            }
        }
    } else {
        if (!d->out_irreps || d->n_out <= 0)
            return fail(why, OEQ_ERR_INVALID_ARG, "an explicit path list needs out_irreps");
        if (d->n_paths <= 0) return fail(why, OEQ_ERR_INVALID_ARG, "n_paths must be positive");
        for (int o = 0; o < d->n_out; ++o) {
            const oeq_irrep &ir = d->out_irreps[o];
            if (ir.mul != p->U && ir.mul != 1)
                return fail(why, OEQ_ERR_UNSUPPORTED, "output blocks must have U channels or one (a channel sum)");
            if (ir.l < 0 || ir.l > kLMax) return fail(why, OEQ_ERR_UNSUPPORTED, "output degree must be in 0..3");
            if (ir.parity != 1 && ir.parity != -1) return fail(why, OEQ_ERR_INVALID_ARG, "parity must be +1 or -1");
            out_lp.push_back({ir.l, ir.parity});
            out_mul.push_back(ir.mul);
        }
        for (int k = 0; k < d->n_paths; ++k) {
            const oeq_path &pa = d->paths[k];
            if (pa.in1 < 0 || pa.in1 >= d->n_x) return fail(why, OEQ_ERR_INVALID_ARG, "path in1 out of range");
            if (pa.in2 < 0 || pa.in2 >= static_cast<int>(p->yb.size()))
                return fail(why, OEQ_ERR_INVALID_ARG, "path Y block out of range");
            if (pa.out < 0 || pa.out >= d->n_out) return fail(why, OEQ_ERR_INVALID_ARG, "path out out of range");
            const int l1 = d->x_irreps[pa.in1].l, l2 = p->yb[pa.in2].l, l3 = out_lp[pa.out].first;
            if (l3 < std::abs(l1 - l2) || l3 > l1 + l2)
                return fail(why, OEQ_ERR_INVALID_ARG, "path violates the triangle rule");
            const int p3 = d->x_irreps[pa.in1].parity * p->yb[pa.in2].parity;
            if (p3 != out_lp[pa.out].second) return fail(why, OEQ_ERR_INVALID_ARG, "path violates parity");
            raw.push_back({pa.in1, pa.in2, pa.out});
        }
    }
    if (raw.empty()) return fail(why, OEQ_ERR_INVALID_ARG, "the descriptor has no paths");
    if (raw.size() > 128) return fail(why, OEQ_ERR_UNSUPPORTED, "more than 128 paths");

    lane = 0;
    row = 0;
    for (size_t o = 0; o < out_lp.size(); ++o) {
        const int l = out_lp[o].first, m = out_mul[o];
        p->ob.push_back({l, out_lp[o].second, lane, row, m, static_cast<int64_t>(p->U) * lane});
        if (m != p->U) p->sum_out = true;
        lane += 2 * l + 1;
        row += static_cast<int64_t>(m) * (2 * l + 1);
    }
    p->NOC = lane;
    p->OD = row;
    p->GOD = static_cast<int64_t>(p->U) * lane;

    p->total_nnz = 0;
    for (const Raw &r : raw) {
        Path pa;
        pa.i1 = r.i1;
        pa.iy = r.iy;
        pa.yoff = p->yb[r.iy].lane_off;
        pa.l1 = p->xb[r.i1].l;
        pa.l2 = p->yb[r.iy].l;
        pa.l3 = p->ob[r.ob].l;
        pa.ob = r.ob;
        pa.parity3 = p->ob[r.ob].parity;
        std::vector<double> t;
        if (!cg_real_table(pa.l1, pa.l2, pa.l3, t)) return fail(why, OEQ_ERR_INVALID_ARG, "invalid path");
        const int n2 = 2 * pa.l2 + 1, n3 = 2 * pa.l3 + 1;
        for (int a = 0; a < 2 * pa.l1 + 1; ++a)
            for (int b = 0; b < n2; ++b)
                for (int c = 0; c < n3; ++c) {
                    const double v = t[(static_cast<size_t>(a) * n2 + b) * n3 + c];
                    if (v != 0.0) pa.nz.push_back({a, b, c, v});
                }
        p->total_nnz += static_cast<int>(pa.nz.size());
        p->paths.push_back(std::move(pa));
    }

    p->uch = (p->U + 63) / 64;
    // m-major atomics need one node row in LDS for the final reorder
    p->xt = p->GXD * (p->dtype == OEQ_F64 ? 8 : 4) <= 65536 && std::getenv("OEQ_NO_XT") == nullptr;
    p->nt_w = std::getenv("OEQ_NO_NT") == nullptr;
    // measured on MI355X: pinning pays for the fp64 forward, not for fp32 or the backward passes
    p->pin_fwd = p->dtype == OEQ_F64;
    p->pin_bwd = false;
    if (const char *e = std::getenv("OEQ_PIN")) {
        p->pin_fwd = std::strchr(e, 'f') != nullptr;
        p->pin_bwd = std::strchr(e, 'b') != nullptr;
    }
    auto waves = [](const char *name, std::pair<int, int> &w) {
        if (const char *e = std::getenv(name)) {
            int a = 0, b = 0;
            if (std::sscanf(e, "%d,%d", &a, &b) == 2 && a >= 1 && b >= a && b <= 8) w = {a, b};
        }
    };
    waves("OEQ_FWD_WAVES", p->fwd_waves);
    waves("OEQ_BWD_WAVES", p->bwd_waves);
    p->fwd_groups = choose_groups(*p, true);
    // measured on MI355X (tiles of 64 edges): the tile form wins for fp64 (medium workload
    // 0.739 against 0.802 ms with the literal form loading two edges ahead) and ties where four
    // or more channel chunks share each edge's rows (wide workload, U = 256: 1.498 against
    // 1.489 ms; 1.62 before the two-edge pipeline); with two chunks in fp32 the literal form is
    // faster (large workload 0.67 against 0.78 ms: the tile form's 172 registers leave two
    // waves per SIMD, and the waves wait while a tile's rows are built)
    p->fwd_lds = p->dtype == OEQ_F64 || p->uch >= 4;
    if (const char *e = std::getenv("OEQ_FWD_LDS")) p->fwd_lds = std::atoi(e) != 0;
    // tiles of 64 edges: one build of the rows per receiver of the degree-56 workloads (wide
    // 1.49 against 1.56 ms with 32); the literal form does not use tiles
    if (p->fwd_lds) p->fwd_tile = 64;
    if (const char *e = std::getenv("OEQ_FWD_TILE")) {
        const int v = std::atoi(e);
        if (v >= 1) p->fwd_tile = v;
    }
    if (const char *e = std::getenv("OEQ_FWD_XCD")) p->fwd_xcd = std::atoi(e) != 0;
    // Loads two edges ahead in the literal forward; one in the VJP. Measured on MI355X (ms,
    // interleaved runs): forward medium fp32 0.350 -> 0.348, and 0.345 with a window of 3 to 4
    // waves per SIMD; large 0.673 -> 0.667 (0.670 with that window); invariant 0.337 -> 0.337
    // (0.333 with it). The VJP two edges ahead: medium 0.815 -> 0.819, large 1.80 -> 1.94,
    // wide 3.78 -> 3.95, medium fp64 1.666 -> 1.652.
    p->fwd_pf = 2;
    if (const char *e = std::getenv("OEQ_FWD_PF")) p->fwd_pf = std::atoi(e) >= 2 ? 2 : 1;
    if (const char *e = std::getenv("OEQ_BWD_PF")) p->bwd_pf = std::atoi(e) >= 2 ? 2 : 1;
    // an output channel sum adds the chunks of a receiver in the workgroup's LDS
    if (p->sum_out) p->fwd_xcd = false;
    // one lane builds one edge's rows: a tile has at most one edge per lane of a group's waves
    p->fwd_tile = std::min(p->fwd_tile, 64 * (p->fwd_xcd ? 1 : p->uch));
    // and the tile's rows stay within 80 KB of LDS (gfx950 gives a workgroup up to 160 KB;
    // 80 KB leaves room for two workgroups per compute unit)
    {
        const int row_bytes = fwd_m_elems(*p) * (p->dtype == OEQ_F64 ? 8 : 4);
        while (p->fwd_tile > 1 && p->fwd_tile * row_bytes > 81920) p->fwd_tile /= 2;
    }
    // the window of 3 to 4 waves for the one-group fp32 literal forward (it fits 170 registers)
    if (p->fwd_waves.first == 0 && std::getenv("OEQ_FWD_WAVES") == nullptr && !p->fwd_lds && p->fwd_pf == 2 &&
        p->fwd_groups.size() == 1 && p->dtype == OEQ_F32)
        p->fwd_waves = {3, 4};
    p->bwd_groups = choose_groups(*p, false);
    p->dbwd_groups = choose_dbwd_groups(*p);
    // The HVP from Y-contracted CG rows, an option (its d_grad_out store leaves out
    // one-channel output blocks, so plans with channel sums keep the fused double backward).
    // Measured on MI355X against the fused kernel: medium fp32 workload 1.02 against 0.80 ms
    // (the fused HVP already moves 5.0 TB/s, the copy rate of the box), large 15.9 against
    // 2.18 ms (the tile form spills: 512 registers against 473 without spills).
    p->hvp_lds = false;
    if (const char *e = std::getenv("OEQ_HVP_LDS")) p->hvp_lds = std::atoi(e) != 0 && !p->sum_out;
    p->hvp_tile = 32;
    if (const char *e = std::getenv("OEQ_HVP_TILE")) {
        const int v = std::atoi(e);
        if (v >= 1) p->hvp_tile = v;
    }
    // one lane builds one edge's rows; the tile's rows stay within 32 KB of LDS
    p->hvp_tile = std::min(p->hvp_tile, 64 * p->uch);
    if (p->hvp_lds) {
        const int row_bytes = hvp_m_elems(*p) * (p->dtype == OEQ_F64 ? 8 : 4);
        while (p->hvp_tile > 1 && p->hvp_tile * row_bytes > 32768) p->hvp_tile /= 2;
    }
    {
        // the radial VJP keeps 2 x 8 x NW more values per lane than the VJP: split until the
        // estimate is under budget (estimates of 358 / 636 / 696 compiled to 394 registers /
        // spills / spills for the medium fp32 / large / medium fp64 configurations)
        const int max_g = std::max(1, 16 / p->uch), f = p->dtype == OEQ_F64 ? 2 : 1;
        auto worst_of = [&](const std::vector<std::vector<int>> &groups) {
            int worst = 0;
            for (const auto &gr : groups)
                worst = std::max(worst, group_registers(*p, gr, false) + 2 * 8 * static_cast<int>(gr.size()) * f);
            return worst;
        };
        for (int g = 1; g <= max_g; ++g) {
            auto cand = partition_paths(*p, false, g);
            p->rad_groups = cand;
            if (worst_of(cand) <= 400 || static_cast<int>(cand.size()) < g) break;
        }
        if (const char *e = std::getenv("OEQ_RAD_GROUPS"))
            p->rad_groups = partition_paths(*p, false, std::max(1, std::min(std::atoi(e), max_g)));
        // a group that is still over the budget spills in the in-kernel pass (the medium fp64
        // configuration's 9-path block: 12 ms against about 3 ms when composed)
        p->rad_compose = worst_of(p->rad_groups) > 400;
        if (const char *e = std::getenv("OEQ_RAD_COMPOSE")) p->rad_compose = std::atoi(e) != 0;
    }
    if (const char *s = std::getenv("OEQ_GY_TILE")) {
        const int v = std::atoi(s);
        if (v >= 1 && v <= 256) p->gy_tile = v;
    }
    if (const char *s = std::getenv("OEQ_DBWD_SPLIT")) {
        const int v = std::atoi(s);
        p->dbwd_split = v < 0 ? 0 : v > 2 ? 2 : v;
    }
    {
        std::vector<bool> used(p->xb.size(), false);
        for (const Path &pa : p->paths) used[pa.i1] = true;
        p->x_unused = std::find(used.begin(), used.end(), false) != used.end();
    }
    // Data-movement model ("source stationary" versus "destination stationary", to be
    // decided from the input and output irreps: [RS] maintainer reply).  Both schedules
    // stream W and Y once; they differ in the per-edge, per-channel elements gathered
    // from or scattered to node rows, with an atomic element weighted kAtomic gathered
    // elements:
    //   forward   receiver-stationary: gather x[s] (NXC)       sender-stationary: atomic add into out[r] (NOC)
    //   VJP       receiver-stationary: gather x[s] + atomic gx   sender-stationary: gather g[r] (NOC)
    // kAtomic is measured on MI355X: 143 M fp32 atomic adds (the sender-stationary
    // forward of the invariant workload) took 0.48 ms where 573 M gathered elements
    // (its receiver-stationary forward) took 0.34 ms, about 6 to 1.
    constexpr double kAtomic = 6.0;
    p->move_fwd[0] = p->NXC;
    p->move_fwd[1] = kAtomic * p->NOC;
    p->move_bwd[0] = (1.0 + kAtomic) * p->NXC;
    p->move_bwd[1] = p->NOC;
    p->sched_fwd = p->move_fwd[1] < p->move_fwd[0] ? 1 : 0;
    p->sched_bwd = p->move_bwd[1] < p->move_bwd[0] ? 1 : 0;
    if (const char *s = std::getenv("OEQ_SCHEDULE")) {  // two letters, forward then VJP: r or s
        if (std::strlen(s) == 2) {
            p->sched_fwd = s[0] == 's';
            p->sched_bwd = s[1] == 's';
        }
    }
    // the sender-stationary passes take U channels in every block
    if (p->bcast_x || p->sum_out) p->sched_fwd = p->sched_bwd = 0;
    return OEQ_OK;
}

}  // namespace oeq
