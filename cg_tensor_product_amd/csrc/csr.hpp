// Graph utilities compiled ahead of time (see csr.hip).
#pragma once

#include <cstddef>
#include <cstdint>

#include <hip/hip_runtime.h>

namespace oeq {

// Scratch bytes of sender_csr (256-byte aligned pieces).
hipError_t sender_csr_workspace(int64_t n_nodes, int64_t n_edges, size_t *bytes);

// srowptr[N+1], sperm[E]: edge ids grouped by sender, increasing within a sender.
hipError_t sender_csr(int64_t n_nodes, int64_t n_edges, const int32_t *src, int32_t *srowptr, int32_t *sperm,
                      void *workspace, hipStream_t stream);

// sender_csr plus sdst[E]: the receiver of edge sperm[k] (the workspace of sender_csr).
hipError_t sender_view(int64_t n_nodes, int64_t n_edges, const int32_t *rowptr, const int32_t *src, int32_t *srowptr,
                       int32_t *sperm, int32_t *sdst, void *workspace, hipStream_t stream);

// Synchronous validation of a receiver CSR; *bad_host receives a bit mask
// (1: rowptr ends, 2: rowptr decreases, 4: src out of range).
hipError_t csr_check(int64_t n_nodes, int64_t n_edges, const int32_t *rowptr, const int32_t *src,
                     hipStream_t stream, int *bad_host);

}  // namespace oeq
