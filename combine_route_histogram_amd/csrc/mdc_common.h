// Shared internals of libmdc (MoE dispatch/combine hot path for AMD Instinct
// MI355X, gfx950): vector types, bf16 helpers, wavefront primitives and the
// host-side shape check.  Included by every kernel source of the library.
#pragma once

#include <hip/hip_runtime.h>

#include <cstdint>
#include <cstring>

#include "mdc.h"

namespace {

typedef unsigned int v4u __attribute__((ext_vector_type(4)));

template <bool NT>
__device__ __forceinline__ void store_v4(v4u* p, v4u v) {
  if (NT) __builtin_nontemporal_store(v, p);
  else *p = v;
}

__device__ __forceinline__ uint64_t lanes_below(int lane) { return (1ull << lane) - 1ull; }

__device__ __forceinline__ float bf16_lo(unsigned w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf16_hi(unsigned w) { return __uint_as_float(w & 0xFFFF0000u); }

// fp32 -> bf16 round to nearest, ties to even (the CAST_RINT of [TL] combine):
// add 0x7FFF plus the lowest kept bit, keep the top 16 bits; NaN -> quiet NaN.
__device__ __forceinline__ unsigned bf16_rne(float f) {
  const unsigned u = __float_as_uint(f);
  if (f != f) return ((u >> 16) & 0x8000u) | 0x7FC0u;
  return (u + 0x7FFFu + ((u >> 16) & 1u)) >> 16;
}

// Loads through addresses rebuilt from integers (readlane / shuffles) would be
// compiled as flat accesses; these keep them in the global address space.
typedef const v4u __attribute__((address_space(1))) g_v4u;
typedef const int32_t __attribute__((address_space(1))) g_i32;
template <bool NT>
__device__ __forceinline__ v4u load_v4(uint64_t addr) {
  if (NT) return __builtin_nontemporal_load(reinterpret_cast<g_v4u*>(addr));
  return *reinterpret_cast<g_v4u*>(addr);
}
__device__ __forceinline__ int32_t load_i32(uint64_t addr) { return *reinterpret_cast<g_i32*>(addr); }

// Inclusive prefix sum over the 64 lanes with DPP lane moves: shifts by
// 1, 2, 4, 8 inside each row of 16 lanes, then row_bcast:15 adds the total of
// rows 0 / 2 to rows 1 / 3 and row_bcast:31 adds the total of rows 0-1 to
// rows 2-3.  Lanes without a source read 0.
__device__ __forceinline__ int wave_inclusive_scan(int v) {
  v += __builtin_amdgcn_update_dpp(0, v, 0x111, 0xF, 0xF, true);  // row_shr:1
  v += __builtin_amdgcn_update_dpp(0, v, 0x112, 0xF, 0xF, true);  // row_shr:2
  v += __builtin_amdgcn_update_dpp(0, v, 0x114, 0xF, 0xF, true);  // row_shr:4
  v += __builtin_amdgcn_update_dpp(0, v, 0x118, 0xF, 0xF, true);  // row_shr:8
  v += __builtin_amdgcn_update_dpp(0, v, 0x142, 0xA, 0xF, false); // row_bcast:15 into rows 1, 3
  v += __builtin_amdgcn_update_dpp(0, v, 0x143, 0xC, 0xF, false); // row_bcast:31 into rows 2, 3
  return v;
}

__device__ __forceinline__ uint64_t shfl64(uint64_t v, int src) {
  const unsigned lo = (unsigned)__shfl((int)(unsigned)v, src, 64);
  const unsigned hi = (unsigned)__shfl((int)(unsigned)(v >> 32), src, 64);
  return ((uint64_t)hi << 32) | lo;
}

__device__ __forceinline__ uint64_t readlane64(uint64_t v, int k) {
  const unsigned lo = (unsigned)__builtin_amdgcn_readlane((int)(unsigned)v, k);
  const unsigned hi = (unsigned)__builtin_amdgcn_readlane((int)(unsigned)(v >> 32), k);
  return ((uint64_t)hi << 32) | lo;
}

// ---------------------------------------------------------------------------
// Host side
// ---------------------------------------------------------------------------
inline size_t round_up(size_t v, size_t a) { return (v + a - 1) / a * a; }
inline bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

// Argument checks shared by every entry point.  MDC_ERR_INVALID: the fields do
// not describe a well-formed problem; MDC_ERR_UNSUPPORTED: a well-formed
// problem outside what this library handles ([CV4] Return Value: 161002 vs
// 561002).
constexpr uint32_t kKnownFlags = MDC_FLAG_FFN_PIPELINE | MDC_FLAG_SPIN_MASK;

mdc_status check_shape(const mdc_shape* sh) {
  if (sh == nullptr) return MDC_ERR_NULLPTR;
  if (sh->world < 1 || sh->rank < 0 || sh->rank >= sh->world) return MDC_ERR_INVALID;
  if (sh->bs < 0 || sh->hidden <= 0 || (sh->hidden % 8) != 0) return MDC_ERR_INVALID;
  if (sh->topk < 1) return MDC_ERR_INVALID;
  if (sh->num_experts <= 0 || (sh->num_experts % sh->world) != 0) return MDC_ERR_INVALID;
  if (sh->capacity < 0) return MDC_ERR_INVALID;
  if (sh->mask_per_route != 0 && sh->mask_per_route != 1) return MDC_ERR_INVALID;
  if (sh->zero_experts < 0 || sh->copy_experts < 0) return MDC_ERR_INVALID;
  if (((uint32_t)sh->flags & ~kKnownFlags) != 0) return MDC_ERR_INVALID;
  if ((int64_t)sh->topk > (int64_t)sh->num_experts + sh->zero_experts + sh->copy_experts) return MDC_ERR_INVALID;
  if (sh->topk > MDC_MAX_TOPK) return MDC_ERR_UNSUPPORTED;
  if (sh->num_experts / sh->world > MDC_MAX_LOCAL_EXPERTS) return MDC_ERR_UNSUPPORTED;
  if (sh->capacity > INT32_MAX) return MDC_ERR_UNSUPPORTED;
  if ((int64_t)sh->world * sh->bs * sh->topk > INT32_MAX) return MDC_ERR_UNSUPPORTED;
  if (sh->world > 65535) return MDC_ERR_UNSUPPORTED;
  if ((int64_t)sh->num_experts + sh->zero_experts + sh->copy_experts > INT32_MAX) return MDC_ERR_UNSUPPORTED;
  return MDC_OK;
}

mdc_status launched() { return hipGetLastError() == hipSuccess ? MDC_OK : MDC_ERR_HIP; }

}  // namespace
