// libmdc_probe: memory-ceiling probes that bench.py times beside the MoE
// dispatch/combine kernels on MI355X (gfx950).  None of them computes any
// part of the method: they move bytes in the access patterns the method's
// kernels use, so that each kernel's time can be set against what the same
// bytes cost in the plainest kernel of that pattern ("PTO MegaMoE Dispatch +
// Combine Fusion Example", Measured Performance: the comparison lives in a
// document not on the page, so the ceilings are measured here).
//
// Every probe runs one wavefront per 64 * V vectors of 16 bytes, with
// non-temporal loads and stores as the product kernels use them.
//   probe_read    read n vectors, fold them into one word per wavefront
//   probe_write   write n vectors of a constant
//   probe_copy    copy n vectors
//   probe_rows_read   read whole rows listed by index (the gather's read half)
//   probe_rows_write  write a constant to whole rows, each source row's
//                     destination rows listed contiguously (the gather's
//                     token-major fan-out write half)
//   probe_rows_fanout read each listed source row once and write it to its
//                     listed destination rows (the gather's data movement
//                     without its metadata work)
//   probe_rows_reduce for each output row, read its listed rows and one more
//                     row of its own and write the XOR of them (the combine's
//                     access pattern without its metadata prologue)

#include <hip/hip_runtime.h>

#include <cstdint>

#include "mdc_probe.h"

namespace {

typedef unsigned int v4u __attribute__((ext_vector_type(4)));

constexpr int kV = 8;   // vectors per lane per wavefront in the streaming probes

__device__ __forceinline__ v4u ld(const v4u* p) { return __builtin_nontemporal_load(p); }
__device__ __forceinline__ void st(v4u* p, v4u v) { __builtin_nontemporal_store(v, p); }

__global__ __launch_bounds__(64) void k_read(const v4u* __restrict__ src, uint64_t n, unsigned* __restrict__ sink) {
  const uint64_t base = (uint64_t)blockIdx.x * 64 * kV + threadIdx.x;
  unsigned a = 0;
#pragma unroll
  for (int u = 0; u < kV; ++u) {
    const uint64_t i = base + (uint64_t)u * 64;
    if (i < n) {
      const v4u v = ld(src + i);
      a ^= v[0] ^ v[1] ^ v[2] ^ v[3];
    }
  }
  // a data-dependent store that (almost) never happens keeps every load live
  if (a == 0x9E3779B9u) sink[blockIdx.x & 1023] = a;
}

__global__ __launch_bounds__(64) void k_write(v4u* __restrict__ dst, uint64_t n, unsigned value) {
  const uint64_t base = (uint64_t)blockIdx.x * 64 * kV + threadIdx.x;
  const v4u v = {value, value ^ 1u, value ^ 2u, value ^ 3u};
#pragma unroll
  for (int u = 0; u < kV; ++u) {
    const uint64_t i = base + (uint64_t)u * 64;
    if (i < n) st(dst + i, v);
  }
}

__global__ __launch_bounds__(64) void k_copy(const v4u* __restrict__ src, v4u* __restrict__ dst, uint64_t n) {
  const uint64_t base = (uint64_t)blockIdx.x * 64 * kV + threadIdx.x;
  v4u v[kV];
#pragma unroll
  for (int u = 0; u < kV; ++u) {
    const uint64_t i = base + (uint64_t)u * 64;
    v[u] = i < n ? ld(src + i) : v4u{0u, 0u, 0u, 0u};
  }
#pragma unroll
  for (int u = 0; u < kV; ++u) {
    const uint64_t i = base + (uint64_t)u * 64;
    if (i < n) st(dst + i, v[u]);
  }
}

// Row probes: one wavefront per (row item, column tile of 64 * VT vectors).
template <int VT>
__global__ __launch_bounds__(64) void k_rows_read(const v4u* __restrict__ src, const int32_t* __restrict__ rows,
                                                  int n_rows, int nvec, int ntiles, unsigned* __restrict__ sink) {
  const int item = blockIdx.x / ntiles, tile = blockIdx.x - item * ntiles;
  if (item >= n_rows) return;
  const v4u* r = src + (int64_t)rows[item] * nvec;
  unsigned a = 0;
#pragma unroll
  for (int u = 0; u < VT; ++u) {
    const int i = tile * 64 * VT + u * 64 + threadIdx.x;
    if (i < nvec) {
      const v4u v = ld(r + i);
      a ^= v[0] ^ v[1] ^ v[2] ^ v[3];
    }
  }
  if (a == 0x9E3779B9u) sink[blockIdx.x & 1023] = a;
}

template <int VT>
__global__ __launch_bounds__(64) void k_rows_write(v4u* __restrict__ dst, const int32_t* __restrict__ off,
                                                   const int32_t* __restrict__ rows, int n_src, int nvec,
                                                   int ntiles) {
  const int item = blockIdx.x / ntiles, tile = blockIdx.x - item * ntiles;
  if (item >= n_src) return;
  v4u v[VT];
#pragma unroll
  for (int u = 0; u < VT; ++u) v[u] = v4u{(unsigned)item, (unsigned)u, threadIdx.x, 7u};
  for (int j = off[item]; j < off[item + 1]; ++j) {
    v4u* d = dst + (int64_t)rows[j] * nvec;
#pragma unroll
    for (int u = 0; u < VT; ++u) {
      const int i = tile * 64 * VT + u * 64 + threadIdx.x;
      if (i < nvec) st(d + i, v[u]);
    }
  }
}

// Read source row src_rows[item] once (tile of 64 * VT vectors) and write it
// to destination rows dst_rows[off[item] .. off[item+1]).
template <int VT>
__global__ __launch_bounds__(64) void k_rows_fanout(const v4u* __restrict__ src, const int32_t* __restrict__ src_rows,
                                                    const int32_t* __restrict__ off, const int32_t* __restrict__ dst_rows,
                                                    v4u* __restrict__ dst, int n_src, int nvec, int ntiles) {
  const int item = blockIdx.x / ntiles, tile = blockIdx.x - item * ntiles;
  if (item >= n_src) return;
  const v4u* r = src + (int64_t)src_rows[item] * nvec;
  v4u v[VT];
#pragma unroll
  for (int u = 0; u < VT; ++u) {
    const int i = tile * 64 * VT + u * 64 + threadIdx.x;
    v[u] = i < nvec ? ld(r + i) : v4u{0u, 0u, 0u, 0u};
  }
  for (int j = off[item]; j < off[item + 1]; ++j) {
    v4u* d = dst + (int64_t)dst_rows[j] * nvec;
#pragma unroll
    for (int u = 0; u < VT; ++u) {
      const int i = tile * 64 * VT + u * 64 + threadIdx.x;
      if (i < nvec) st(d + i, v[u]);
    }
  }
}

// For output row t: read rows[t*K .. t*K + K) (entries < 0 are absent) of src
// and row t of own, write their XOR to row t of dst.  One vector per lane;
// KM >= K row slots, all loads issued before the first is used.
template <int KM>
__global__ __launch_bounds__(64) void k_rows_reduce(const v4u* __restrict__ src, const int32_t* __restrict__ rows,
                                                    int K, const v4u* __restrict__ own, v4u* __restrict__ dst,
                                                    int n_out, int nvec, int ntiles) {
  const int t = blockIdx.x / ntiles, tile = blockIdx.x - t * ntiles;
  if (t >= n_out) return;
  const int i = tile * 64 + threadIdx.x;
  const int r = (int)threadIdx.x < K ? rows[(int64_t)t * K + threadIdx.x] : -1;
  v4u v[KM];
#pragma unroll
  for (int k = 0; k < KM; ++k) {
    const int rk = __shfl(r, k, 64);
    v[k] = (k < K && rk >= 0 && i < nvec) ? ld(src + (int64_t)rk * nvec + i) : v4u{0u, 0u, 0u, 0u};
  }
  v4u acc = i < nvec ? ld(own + (int64_t)t * nvec + i) : v4u{0u, 0u, 0u, 0u};
#pragma unroll
  for (int k = 0; k < KM; ++k) acc ^= v[k];
  if (i < nvec) st(dst + (int64_t)t * nvec + i, acc);
}

int status_of(hipError_t e) { return e == hipSuccess ? 0 : 1; }

}  // namespace

extern "C" {

int mdc_probe_read(const void* src, uint64_t bytes, void* sink, void* stream) {
  if (src == nullptr || sink == nullptr || (bytes & 15) != 0) return 2;
  const uint64_t n = bytes / 16;
  if (n == 0) return 0;
  (void)hipGetLastError();
  hipLaunchKernelGGL(k_read, dim3((unsigned)((n + 64 * kV - 1) / (64 * kV))), dim3(64), 0, (hipStream_t)stream,
                     (const v4u*)src, n, (unsigned*)sink);
  return status_of(hipGetLastError());
}

int mdc_probe_write(void* dst, uint64_t bytes, uint32_t value, void* stream) {
  if (dst == nullptr || (bytes & 15) != 0) return 2;
  const uint64_t n = bytes / 16;
  if (n == 0) return 0;
  (void)hipGetLastError();
  hipLaunchKernelGGL(k_write, dim3((unsigned)((n + 64 * kV - 1) / (64 * kV))), dim3(64), 0, (hipStream_t)stream,
                     (v4u*)dst, n, value);
  return status_of(hipGetLastError());
}

int mdc_probe_copy(const void* src, void* dst, uint64_t bytes, void* stream) {
  if (src == nullptr || dst == nullptr || (bytes & 15) != 0) return 2;
  const uint64_t n = bytes / 16;
  if (n == 0) return 0;
  (void)hipGetLastError();
  hipLaunchKernelGGL(k_copy, dim3((unsigned)((n + 64 * kV - 1) / (64 * kV))), dim3(64), 0, (hipStream_t)stream,
                     (const v4u*)src, (v4u*)dst, n);
  return status_of(hipGetLastError());
}

int mdc_probe_rows_read(const void* src, const int32_t* rows, int32_t n_rows, int32_t row_bytes, void* sink,
                        void* stream) {
  if (src == nullptr || rows == nullptr || sink == nullptr || n_rows < 0 || row_bytes <= 0 || (row_bytes & 15))
    return 2;
  if (n_rows == 0) return 0;
  const int nvec = row_bytes / 16;
  const int ntiles = (nvec + 64 * 7 - 1) / (64 * 7);
  (void)hipGetLastError();
  hipLaunchKernelGGL(k_rows_read<7>, dim3((unsigned)((int64_t)n_rows * ntiles)), dim3(64), 0, (hipStream_t)stream,
                     (const v4u*)src, rows, n_rows, nvec, ntiles, (unsigned*)sink);
  return status_of(hipGetLastError());
}

int mdc_probe_rows_write(void* dst, const int32_t* offsets, const int32_t* rows, int32_t n_src, int32_t row_bytes,
                         void* stream) {
  if (dst == nullptr || offsets == nullptr || rows == nullptr || n_src < 0 || row_bytes <= 0 || (row_bytes & 15))
    return 2;
  if (n_src == 0) return 0;
  const int nvec = row_bytes / 16;
  const int ntiles = (nvec + 64 * 7 - 1) / (64 * 7);
  (void)hipGetLastError();
  hipLaunchKernelGGL(k_rows_write<7>, dim3((unsigned)((int64_t)n_src * ntiles)), dim3(64), 0, (hipStream_t)stream,
                     (v4u*)dst, offsets, rows, n_src, nvec, ntiles);
  return status_of(hipGetLastError());
}

int mdc_probe_rows_fanout(const void* src, const int32_t* src_rows, const int32_t* offsets, const int32_t* dst_rows,
                          void* dst, int32_t n_src, int32_t row_bytes, void* stream) {
  if (src == nullptr || src_rows == nullptr || offsets == nullptr || dst_rows == nullptr || dst == nullptr ||
      n_src < 0 || row_bytes <= 0 || (row_bytes & 15))
    return 2;
  if (n_src == 0) return 0;
  const int nvec = row_bytes / 16;
  const int ntiles = (nvec + 64 * 7 - 1) / (64 * 7);
  (void)hipGetLastError();
  hipLaunchKernelGGL(k_rows_fanout<7>, dim3((unsigned)((int64_t)n_src * ntiles)), dim3(64), 0, (hipStream_t)stream,
                     (const v4u*)src, src_rows, offsets, dst_rows, (v4u*)dst, n_src, nvec, ntiles);
  return status_of(hipGetLastError());
}

int mdc_probe_rows_reduce(const void* src, const int32_t* rows, int32_t k, const void* own, void* dst, int32_t n_out,
                          int32_t row_bytes, void* stream) {
  if (src == nullptr || rows == nullptr || own == nullptr || dst == nullptr || n_out < 0 || k < 1 || k > 16 ||
      row_bytes <= 0 || (row_bytes & 15))
    return 2;
  if (n_out == 0) return 0;
  const int nvec = row_bytes / 16;
  const int ntiles = (nvec + 63) / 64;
  (void)hipGetLastError();
  const dim3 grid((unsigned)((int64_t)n_out * ntiles));
  if (k <= 8)
    hipLaunchKernelGGL(k_rows_reduce<8>, grid, dim3(64), 0, (hipStream_t)stream, (const v4u*)src, rows, k,
                       (const v4u*)own, (v4u*)dst, n_out, nvec, ntiles);
  else
    hipLaunchKernelGGL(k_rows_reduce<16>, grid, dim3(64), 0, (hipStream_t)stream, (const v4u*)src, rows, k,
                       (const v4u*)own, (v4u*)dst, n_out, nvec, ntiles);
  return status_of(hipGetLastError());
}

}  // extern "C"
