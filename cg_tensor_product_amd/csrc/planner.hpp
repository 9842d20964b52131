// Host-side plan of a channel-wise (UVU) CG tensor-product convolution: the
// validated irreps, the path list with its sparse real-basis CG tables, the row
// layouts, the emitted HIP source and the runtime-compiled code object.
#pragma once

#include <cstdint>
#include <map>
#include <mutex>
#include <string>
#include <vector>

#include <hip/hip_runtime.h>

#include "oeq.h"

namespace oeq {

constexpr int kLMax = 3;

// Dense real-basis CG table for (l1, l2, l3) (see cg_tables.cpp); false outside
// the triangle rule or l > 3.
bool cg_real_table(int l1, int l2, int l3, std::vector<double> &out);

struct NonZero {
    int m1, m2, m3;  // 0-based: m + l
    double c;
};

struct Path {
    int i1;          // x block
    int iy;          // Y block
    int yoff;        // offset of the Y block in a Y row
    int l1, l2, l3;
    int ob;          // output block
    int parity3;
    std::vector<NonZero> nz;
};

struct Block {
    int l, parity;
    int lane_off;    // offset of this block among one channel's values (sum of 2l+1 before it)
    int64_t row_off; // offset of this block in a node row (the sum of mul * (2l+1) before it)
    int mul = 0;     // channels: U, or 1 for an x block broadcast against the U channels or an
                     // output block that sums them
    int64_t exp_off = 0;  // offset in a row with U channels in every block (U * lane_off)
};

// Kernels of one compiled module, on one device.
struct DeviceModule {
    hipModule_t module = nullptr;
    std::map<std::string, hipFunction_t> fn;
};

struct oeq_plan_impl;

}  // namespace oeq

struct oeq_plan {
    oeq_dtype dtype;
    int U = 0;
    int L = 0;                  // largest Y degree
    int YD = 0;                 // Y row width: sum of 2l+1 over the Y blocks
    bool y_natural = true;      // every Y block has parity (-1)^l (spherical harmonics can fill it)
    int NXC = 0, NOC = 0;       // per-channel x and output widths
    int64_t XD = 0, OD = 0;     // node row widths
    // Rows with U channels in every block: the kernels write x-gradient rows this way and a
    // fold sums the channels of the one-channel x blocks (GXD > XD only then).  An output
    // block of one channel is summed over the channels in the forward itself.
    int64_t GXD = 0, GOD = 0;
    bool bcast_x = false;       // some x block has one channel and U > 1
    bool sum_out = false;       // some output block has one channel and U > 1
    std::vector<oeq::Block> xb, ob, yb;  // yb: lane_off = offset in a Y row
    std::vector<oeq::Path> paths;
    int total_nnz = 0;

    // Launch shape.
    int uch = 1;                // 64-channel chunks (waves per receiver)
    int gy_tile = 32;           // edges per LDS gY flush in the backward kernels
    int dbwd_split = -1;        // double backward: 0 one fused pass; 1 split by output; 2 also one d_Y/d_x pass per tangent; -1 the first that does not spill
    bool xt = false;            // x-gradient atomics use an m-major row (needs the row in LDS)
    bool x_unused = false;      // some x block feeds no path (its gradient is zero)
    // Schedule the data-movement model prefers for each pass (0 receiver-, 1 sender-stationary)
    // and the per-edge bytes it compares.
    int sched_fwd = 0, sched_bwd = 0;
    double move_fwd[2] = {0, 0}, move_bwd[2] = {0, 0};
    bool nt_w = true;           // non-temporal loads/stores for W and its gradients
    // forward with the CG tables contracted with Y per edge tile in LDS (M[e] = C . Y[e],
    // built with one lane per edge), so each lane does |M| + min(n1, n3) multiply-adds per
    // path instead of the x-Y products plus every non-zero plus n3
    bool fwd_lds = false;
    int fwd_tile = 32;          // edges per LDS tile of M rows (capped by the LDS budget)
    int fwd_pf = 1;             // edges the literal forward loads ahead of the one it computes
    int bwd_pf = 1;             // the same for the VJP
    // the HVP (tangent on x only) from Y-contracted CG rows in LDS per edge tile: d_grad_out
    // and d_W share the forward of the tangent, t = M^T v, instead of the x-Y products
    bool hvp_lds = false;
    int hvp_tile = 32;          // edges per HVP tile (at most one per lane of the workgroup)
    // forward workgroups of one 64-channel chunk, mapped so that each chunk stays on the
    // same XCDs (their L2 caches then hold the x rows of one chunk)
    bool fwd_xcd = false;
    // keep the software-pipelined loads ahead of the arithmetic (forward, backward passes)
    bool pin_fwd = false, pin_bwd = false;
    std::pair<int, int> fwd_waves{0, 0}, bwd_waves{0, 0};  // (min, max) waves per SIMD; 0 = compiler default
    // Path groups: one wave computes one group for 64 channels of a receiver.
    std::vector<std::vector<int>> fwd_groups, bwd_groups;
    // path groups of the double-backward kernels with more than the gg_x tangent (the HVP,
    // gg_x alone, keeps bwd_groups)
    std::vector<std::vector<int>> dbwd_groups;
    // groups of the VJP that forms the radial weights in the kernel (it also holds the
    // hidden-width slices of W2 and of the W2 gradient per lane)
    std::vector<std::vector<int>> rad_groups;
    // the VJP with in-kernel radial weights runs as W = h W2, the convolution VJP and two
    // dense products instead (its groups do not fit registers)
    bool rad_compose = false;

    std::string source;         // emitted HIP source
    std::vector<char> code;     // gfx950 code object
    std::string code_key;       // cache key (hash of source + options)

    std::mutex mu;
    std::map<int, oeq::DeviceModule> modules;  // per device id
};

namespace oeq {

// Validates the descriptor and fills the structural part of the plan (paths,
// tables, layouts).  Returns OEQ_OK or an error with a message in *why.
oeq_status plan_build(const oeq_tp_desc *d, oeq_plan *p, std::string *why);

// Elements of one edge's Y-contracted CG rows over all forward groups (the LDS forward).
int fwd_m_elems(const oeq_plan &p);
// Largest M row over the backward groups (the tile-form HVP).
int hvp_m_elems(const oeq_plan &p);

// Emits the HIP source of every kernel of the plan.
std::string emit_source(const oeq_plan &p);

// Compiles p.source with hipRTC (or loads it from the on-disk cache); with
// cache_only, a code object missing from the cache is an OEQ_ERR_JIT instead.
oeq_status jit_compile(oeq_plan &p, std::string *why, bool cache_only = false);

// Loads the module on the current device (once) and returns the kernel.
oeq_status get_kernel(oeq_plan &p, const char *name, hipFunction_t *fn, std::string *why);

// Whether the plan's module is already loaded on device `dev` (a load allocates device memory).
bool module_loaded(oeq_plan &p, int dev);

}  // namespace oeq
