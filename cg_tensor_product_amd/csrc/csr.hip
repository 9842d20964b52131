// Graph utilities compiled ahead of time (they do not depend on the irreps):
// the sender CSR (a stable sort of edge ids by sender) used by the deterministic
// x-gradient, and a synchronous validator of a receiver CSR.
//
// The sender CSR is the transpose of the receiver-sorted edge list: edge ids
// grouped by sender, increasing inside a group.  A stable LSD radix sort of
// (src[e], e) pairs yields exactly that order; srowptr[s] is then the first
// position whose sorted key is >= s.
#include <hip/hip_runtime.h>

#include <rocprim/device/device_radix_sort.hpp>
#include <rocprim/iterator/counting_iterator.hpp>

#include "csr.hpp"

namespace oeq {

namespace {

unsigned key_bits(int64_t n_nodes) {
    unsigned b = 1;
    while (b < 31 && (int64_t(1) << b) < n_nodes) ++b;
    return b;
}

__global__ void __launch_bounds__(256) k_sender_rowptr(const int *__restrict__ sorted, int n_edges, int n_nodes,
                                                      int *__restrict__ srowptr) {
    const int s = blockIdx.x * blockDim.x + threadIdx.x;
    if (s > n_nodes) return;
    int lo = 0, hi = n_edges;  // first position with sorted[pos] >= s
    while (lo < hi) {
        const int mid = lo + (hi - lo) / 2;
        if (sorted[mid] < s)
            lo = mid + 1;
        else
            hi = mid;
    }
    srowptr[s] = lo;
}

__global__ void __launch_bounds__(256) k_csr_check(const int *__restrict__ rowptr, const int *__restrict__ src,
                                                  int n_nodes, int n_edges, int *__restrict__ bad) {
    const int64_t i = int64_t(blockIdx.x) * blockDim.x + threadIdx.x;
    if (i == 0 && (rowptr[0] != 0 || rowptr[n_nodes] != n_edges)) atomicOr(bad, 1);
    if (i < n_nodes && rowptr[i + 1] < rowptr[i]) atomicOr(bad, 2);
    if (i < n_edges && (src[i] < 0 || src[i] >= n_nodes)) atomicOr(bad, 4);
}

constexpr size_t kAlign = 256;
size_t up(size_t v) { return (v + kAlign - 1) / kAlign * kAlign; }

}  // namespace

hipError_t sender_csr_workspace(int64_t n_nodes, int64_t n_edges, size_t *bytes) {
    size_t temp = 0;
    const hipError_t e = rocprim::radix_sort_pairs(
        nullptr, temp, static_cast<const int *>(nullptr), static_cast<int *>(nullptr),
        rocprim::counting_iterator<int>(0), static_cast<int *>(nullptr), static_cast<unsigned>(n_edges), 0,
        key_bits(n_nodes));
    *bytes = up(sizeof(int) * static_cast<size_t>(n_edges > 0 ? n_edges : 1)) + up(temp);
    return e;
}

hipError_t sender_csr(int64_t n_nodes, int64_t n_edges, const int32_t *src, int32_t *srowptr, int32_t *sperm,
                      void *workspace, hipStream_t stream) {
    char *ws = static_cast<char *>(workspace);
    int *sorted = reinterpret_cast<int *>(ws);
    char *temp = ws + up(sizeof(int) * static_cast<size_t>(n_edges > 0 ? n_edges : 1));
    if (n_edges > 0) {
        size_t temp_bytes = 0;
        hipError_t e = rocprim::radix_sort_pairs(
            nullptr, temp_bytes, src, sorted, rocprim::counting_iterator<int>(0), sperm,
            static_cast<unsigned>(n_edges), 0, key_bits(n_nodes), stream);
        if (e != hipSuccess) return e;
        e = rocprim::radix_sort_pairs(temp, temp_bytes, src, sorted, rocprim::counting_iterator<int>(0), sperm,
                                      static_cast<unsigned>(n_edges), 0, key_bits(n_nodes), stream);
        if (e != hipSuccess) return e;
    }
    const int threads = 256;
    const int blocks = static_cast<int>((n_nodes + 1 + threads - 1) / threads);
    hipLaunchKernelGGL(k_sender_rowptr, dim3(blocks), dim3(threads), 0, stream, sorted,
                       static_cast<int>(n_edges), static_cast<int>(n_nodes), srowptr);
    return hipGetLastError();
}

hipError_t csr_check(int64_t n_nodes, int64_t n_edges, const int32_t *rowptr, const int32_t *src,
                     hipStream_t stream, int *bad_host) {
    int *bad = nullptr;
    hipError_t e = hipMalloc(&bad, sizeof(int));
    if (e != hipSuccess) return e;
    e = hipMemsetAsync(bad, 0, sizeof(int), stream);
    const int64_t n = (n_nodes > n_edges ? n_nodes : n_edges) + 1;
    const int threads = 256;
    const int blocks = static_cast<int>((n + threads - 1) / threads);
    if (e == hipSuccess) {
        hipLaunchKernelGGL(k_csr_check, dim3(blocks), dim3(threads), 0, stream, rowptr, src,
                           static_cast<int>(n_nodes), static_cast<int>(n_edges), bad);
        e = hipGetLastError();
    }
    if (e == hipSuccess) e = hipMemcpyAsync(bad_host, bad, sizeof(int), hipMemcpyDeviceToHost, stream);
    if (e == hipSuccess) e = hipStreamSynchronize(stream);
    (void)hipFree(bad);
    return e;
}

}  // namespace oeq
