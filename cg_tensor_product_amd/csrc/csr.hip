// Graph utilities compiled ahead of time (they do not depend on the irreps):
// the sender CSR used by the deterministic x-gradient, and a synchronous
// validator of a receiver CSR.
//
// The sender CSR is the transpose of the receiver-sorted edge list: edge ids
// grouped by sender, increasing inside a group (a stable counting sort by
// sender).  It is built with kernels only (no memset or copy nodes, so a caller
// may capture it in a HIP graph):
//   1. cursor[s] = 0; count[s] += 1 per edge (integer atomics: exact);
//   2. srowptr = exclusive prefix sum of count (one workgroup);
//   3. each edge takes a slot in its sender's bucket through an atomic cursor;
//   4. each bucket is put in increasing edge order by ranking: the slot of edge
//      e is the number of edges in the bucket with a smaller id.
// Steps 3-4 give the same array on every run whatever order the atomics take.
#include <hip/hip_runtime.h>

#include "csr.hpp"

namespace oeq {

namespace {

constexpr int kScanThreads = 1024;

__global__ void __launch_bounds__(256) k_zero_i32(int *__restrict__ p, int64_t n) {
    for (int64_t i = int64_t(blockIdx.x) * blockDim.x + threadIdx.x; i < n; i += int64_t(gridDim.x) * blockDim.x)
        p[i] = 0;
}

__global__ void __launch_bounds__(256) k_count(const int *__restrict__ src, int n_edges, int *__restrict__ count) {
    for (int e = blockIdx.x * blockDim.x + threadIdx.x; e < n_edges; e += gridDim.x * blockDim.x)
        atomicAdd(&count[src[e]], 1);
}

// Exclusive prefix sum of count[0..n) into rowptr[0..n]; one workgroup: each
// thread sums a contiguous chunk, the chunk totals are scanned in LDS, then each
// thread writes its chunk's running sums.
__global__ void __launch_bounds__(kScanThreads) k_scan(const int *__restrict__ count, int n, int *__restrict__ rowptr) {
    __shared__ int part[kScanThreads];
    const int t = threadIdx.x;
    const int chunk = (n + kScanThreads - 1) / kScanThreads;
    const int a = min(n, t * chunk), b = min(n, a + chunk);
    int s = 0;
    for (int i = a; i < b; ++i) s += count[i];
    part[t] = s;
    __syncthreads();
    for (int off = 1; off < kScanThreads; off <<= 1) {  // inclusive Hillis-Steele scan
        const int v = t >= off ? part[t - off] : 0;
        __syncthreads();
        part[t] += v;
        __syncthreads();
    }
    int run = t == 0 ? 0 : part[t - 1];
    for (int i = a; i < b; ++i) {
        rowptr[i] = run;
        run += count[i];
    }
    if (t == kScanThreads - 1) rowptr[n] = part[kScanThreads - 1];
}

__global__ void __launch_bounds__(256) k_place(const int *__restrict__ src, int n_edges,
                                               const int *__restrict__ rowptr, int *__restrict__ cursor,
                                               int *__restrict__ tmp) {
    for (int e = blockIdx.x * blockDim.x + threadIdx.x; e < n_edges; e += gridDim.x * blockDim.x) {
        const int s = src[e];
        tmp[rowptr[s] + atomicAdd(&cursor[s], 1)] = e;
    }
}

// One wave per sender bucket: edge ids are distinct, so the number of smaller
// ids in the bucket is the edge's position in increasing order.
__global__ void __launch_bounds__(256) k_rank(const int *__restrict__ rowptr, int n_nodes,
                                              const int *__restrict__ tmp, int *__restrict__ perm) {
    const int lane = threadIdx.x & 63;
    for (int s = blockIdx.x * 4 + (threadIdx.x >> 6); s < n_nodes; s += gridDim.x * 4) {
        const int a = rowptr[s], d = rowptr[s + 1] - a;
        for (int i = lane; i < d; i += 64) {
            const int v = tmp[a + i];
            int rank = 0;
            for (int j = 0; j < d; ++j) rank += tmp[a + j] < v;
            perm[a + rank] = v;
        }
    }
}

// The receiver of each edge in sender order: the receiver-CSR row r holding edge
// e = sperm[k], i.e. the largest r with rowptr[r] <= e (rows may be empty).
__global__ void __launch_bounds__(256) k_sdst(const int *__restrict__ rowptr, int n_nodes,
                                              const int *__restrict__ sperm, int n_edges, int *__restrict__ sdst) {
    for (int k = blockIdx.x * blockDim.x + threadIdx.x; k < n_edges; k += gridDim.x * blockDim.x) {
        const int e = sperm[k];
        int lo = 0, hi = n_nodes;  // rowptr[lo] <= e < rowptr[hi]
        while (hi - lo > 1) {
            const int mid = lo + (hi - lo) / 2;
            if (rowptr[mid] <= e)
                lo = mid;
            else
                hi = mid;
        }
        sdst[k] = lo;
    }
}

__global__ void __launch_bounds__(256) k_csr_check(const int *__restrict__ rowptr, const int *__restrict__ src,
                                                  int n_nodes, int n_edges, int *__restrict__ bad) {
    const int64_t n = n_nodes > n_edges ? n_nodes : n_edges;
    for (int64_t i = int64_t(blockIdx.x) * blockDim.x + threadIdx.x; i < n + 1; i += int64_t(gridDim.x) * blockDim.x) {
        if (i == 0 && (rowptr[0] != 0 || rowptr[n_nodes] != n_edges)) atomicOr(bad, 1);
        if (i < n_nodes && rowptr[i + 1] < rowptr[i]) atomicOr(bad, 2);
        if (i < n_edges && (src[i] < 0 || src[i] >= n_nodes)) atomicOr(bad, 4);
    }
}

constexpr size_t kAlign = 256;
size_t up(size_t v) { return (v + kAlign - 1) / kAlign * kAlign; }

unsigned grid_for(int64_t n, int64_t per_block) {
    int64_t g = (n + per_block - 1) / per_block;
    if (g < 1) g = 1;
    if (g > 65536) g = 65536;
    return static_cast<unsigned>(g);
}

}  // namespace

hipError_t sender_csr_workspace(int64_t n_nodes, int64_t n_edges, size_t *bytes) {
    // count / cursor [N], bucket slots [E]
    *bytes = up(sizeof(int) * static_cast<size_t>(n_nodes > 0 ? n_nodes : 1)) * 2 +
             up(sizeof(int) * static_cast<size_t>(n_edges > 0 ? n_edges : 1));
    return hipSuccess;
}

hipError_t sender_csr(int64_t n_nodes, int64_t n_edges, const int32_t *src, int32_t *srowptr, int32_t *sperm,
                      void *workspace, hipStream_t stream) {
    char *ws = static_cast<char *>(workspace);
    const size_t nb = up(sizeof(int) * static_cast<size_t>(n_nodes > 0 ? n_nodes : 1));
    int *count = reinterpret_cast<int *>(ws);
    int *cursor = reinterpret_cast<int *>(ws + nb);
    int *tmp = reinterpret_cast<int *>(ws + 2 * nb);
    const int N = static_cast<int>(n_nodes), E = static_cast<int>(n_edges);
    hipLaunchKernelGGL(k_zero_i32, dim3(grid_for(2 * nb / sizeof(int), 256)), dim3(256), 0, stream, count,
                       static_cast<int64_t>(2 * nb / sizeof(int)));
    if (E > 0) hipLaunchKernelGGL(k_count, dim3(grid_for(E, 256)), dim3(256), 0, stream, src, E, count);
    hipLaunchKernelGGL(k_scan, dim3(1), dim3(kScanThreads), 0, stream, count, N, srowptr);
    if (E > 0) {
        hipLaunchKernelGGL(k_place, dim3(grid_for(E, 256)), dim3(256), 0, stream, src, E, srowptr, cursor, tmp);
        hipLaunchKernelGGL(k_rank, dim3(grid_for(N, 4)), dim3(256), 0, stream, srowptr, N, tmp, sperm);
    }
    return hipGetLastError();
}

hipError_t sender_view(int64_t n_nodes, int64_t n_edges, const int32_t *rowptr, const int32_t *src, int32_t *srowptr,
                       int32_t *sperm, int32_t *sdst, void *workspace, hipStream_t stream) {
    hipError_t e = sender_csr(n_nodes, n_edges, src, srowptr, sperm, workspace, stream);
    if (e != hipSuccess || n_edges == 0) return e;
    hipLaunchKernelGGL(k_sdst, dim3(grid_for(n_edges, 256)), dim3(256), 0, stream, rowptr,
                       static_cast<int>(n_nodes), sperm, static_cast<int>(n_edges), sdst);
    return hipGetLastError();
}

hipError_t csr_check(int64_t n_nodes, int64_t n_edges, const int32_t *rowptr, const int32_t *src,
                     hipStream_t stream, int *bad_host) {
    int *bad = nullptr;
    hipError_t e = hipMalloc(&bad, sizeof(int));
    if (e != hipSuccess) return e;
    hipLaunchKernelGGL(k_zero_i32, dim3(1), dim3(256), 0, stream, bad, int64_t(1));
    const int64_t n = (n_nodes > n_edges ? n_nodes : n_edges) + 1;
    hipLaunchKernelGGL(k_csr_check, dim3(grid_for(n, 256)), dim3(256), 0, stream, rowptr, src,
                       static_cast<int>(n_nodes), static_cast<int>(n_edges), bad);
    e = hipGetLastError();
    if (e == hipSuccess) e = hipMemcpyAsync(bad_host, bad, sizeof(int), hipMemcpyDeviceToHost, stream);
    if (e == hipSuccess) e = hipStreamSynchronize(stream);
    (void)hipFree(bad);
    return e;
}

}  // namespace oeq
