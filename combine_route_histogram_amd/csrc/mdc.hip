// libmdc: MoE dispatch/combine hot path for AMD Instinct MI355X (gfx950).
//
// Kernels (one GPU's share; the W expert-parallel ranks are virtual buffers):
//   k_route_rank      per group of one source's routes: local-route filter,
//                     wavefront-ballot multi-split rank within (source, local
//                     expert), group histogram.  (mdc_dispatch_layout)
//   k_dispatch_gather one wavefront per (source token, column tile): scans the
//                     group histograms in-wavefront to place the token's
//                     routes, reads its row tile once and writes it to each of
//                     its rows on this rank, with the (src, token, k) triplets,
//                     the route -> row inverse index, epRecvCounts and
//                     expertTokenNums.  (mdc_dispatch_gather)
//   k_combine         one wavefront per (token, column tile) of the combining
//                     rank: reads the token's present expert rows (and the
//                     shared-expert row), accumulates in fp32 in ascending k,
//                     rounds to bf16 nearest-even.  (mdc_combine)
//
// Sources: "dispatch_combine_shmem.py" (TileLang-Ascend example),
// moe_dispatch_kernel / moe_combine_kernel; "aclnnMoeDistributeCombineV4",
// Function formula and Function Prototype; "PTO MegaMoE Dispatch + Combine
// Fusion Example", FrontReorder / Dispatch / Combine / Unpermute stages.
//
// Built with -ffp-contract=off: the combine's products and sums are rounded
// to fp32 one by one, in the order the combine formula lists them.

#include <hip/hip_runtime.h>

#include <cstdint>
#include <cstring>

#include "mdc.h"

namespace {

typedef unsigned int v4u __attribute__((ext_vector_type(4)));

// Build-time tile shapes (16-byte vectors per lane per row tile).
#ifndef MDC_GATHER_VEC
#define MDC_GATHER_VEC 8
#endif
#ifndef MDC_COMBINE_VEC
#define MDC_COMBINE_VEC 1
#endif
// Cache policy per kernel (1 = non-temporal).  Measured on MI355X over whole
// dispatch+combine steps: non-temporal row loads and stores in both kernels
// give the shortest step (the two kernels share the Infinity Cache, so each
// one's policy also moves the other's time).
// Wavefronts per workgroup (each wavefront handles its own row tile).
#ifndef MDC_GATHER_WAVES
#define MDC_GATHER_WAVES 1
#endif
#ifndef MDC_COMBINE_WAVES
#define MDC_COMBINE_WAVES 1
#endif
#ifndef MDC_GATHER_NT_LOADS
#define MDC_GATHER_NT_LOADS 1
#endif
#ifndef MDC_GATHER_NT_STORES
#define MDC_GATHER_NT_STORES 1
#endif
#ifndef MDC_COMBINE_NT_LOADS
#define MDC_COMBINE_NT_LOADS 1
#endif
#ifndef MDC_COMBINE_NT_STORES
#define MDC_COMBINE_NT_STORES 1
#endif
#ifndef MDC_GROUP_ROUTES
#define MDC_GROUP_ROUTES 2048
#endif
#ifndef MDC_SCAN_IPL
#define MDC_SCAN_IPL 16
#endif
constexpr int kGroupRoutes = MDC_GROUP_ROUTES;  // routes of one source ranked by one k_route_rank workgroup
constexpr int kScanIPL = MDC_SCAN_IPL;           // group counters per lane per scan chunk
constexpr int kScanChunk = 64 * kScanIPL;

// Group counters are scanned in chunks of kScanChunk, lane l taking the
// kScanIPL consecutive counters l*kScanIPL.. of a chunk.  They are stored
// transposed inside each chunk (counter j of lane l at j*64 + l) so that the
// j-th load of all 64 lanes reads 64 consecutive words.
__host__ __device__ __forceinline__ int counter_slot(int i) {
  const int c0 = i - i % kScanChunk;
  const int r = i - c0;
  return c0 + (r % kScanIPL) * 64 + r / kScanIPL;
}
constexpr int kGatherVec = MDC_GATHER_VEC;
static_assert(kGatherVec >= 1 && kGatherVec <= 8, "gather tiles hold 1..8 vectors per lane");
constexpr int kCombineVec = MDC_COMBINE_VEC;

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
// a1 + a3 (ranks): route filter, histogram and stable rank within a group.
//
// A group is TPG = floor(4096 / K) consecutive tokens of one source rank; one
// workgroup walks its routes in flattened (t, k) order, one route per thread
// per step.  A route's key is its local expert le = e - d*L when it is sent
// to rank d (active token, 0 <= e < E, e / L == d), else L.  Inside a
// wavefront, one ballot per key bit isolates the lanes holding the same key
// (a multi-split); the rank is the count of those lanes below.  Wavefront
// counts are prefixed in LDS in wavefront order on top of the counts carried
// from earlier steps, so rank = number of earlier routes of this source and
// group with the same expert ([TL] send loop: rank-within-expert counts the
// earlier equal ids).
//
// P[f] = le | (rank << 16) for a route sent to d, else -1.
// cnt[(le*W + s)*G + g] = routes of group g of source s sent to local expert le.
// ---------------------------------------------------------------------------
__global__ __launch_bounds__(1024) void k_route_rank(
    const int32_t* __restrict__ ids, const uint8_t* __restrict__ mask,
    int32_t* __restrict__ P, int32_t* __restrict__ cnt,
    int BS, int K, int E, int L, int d, int W, int TPG, int G, int mask_per_route) {
  extern __shared__ int32_t sm[];  // carry[L], wave_cnt[nw][L]
  const int nw = blockDim.x >> 6;
  int32_t* carry = sm;
  int32_t* wave_cnt = sm + L;
  const int s = blockIdx.y;
  const int g = blockIdx.x;
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wv = tid >> 6;
  const int t_begin = g * TPG;
  const int t_end = min(BS, t_begin + TPG);
  const int n_routes = (t_end - t_begin) * K;
  const int64_t f_base = ((int64_t)s * BS + t_begin) * K;
  const int nbits = 32 - __clz(L);

  // Every key of the group is computed up front so that the id loads of all
  // steps are in flight together (a group holds at most kGroupRoutes routes).
  constexpr int kMaxSteps = kGroupRoutes / 256;
  int keys[kMaxSteps];
#pragma unroll
  for (int i = 0; i < kMaxSteps; ++i) {
    const int f = i * (int)blockDim.x + tid;
    int key = L;
    if (f < n_routes) {
      const int t = t_begin + f / K;
      const int e = ids[f_base + f];
      const bool active = (mask == nullptr) ||
                          (mask[mask_per_route ? f_base + f : (int64_t)s * BS + t] != 0);
      const int q = e - d * L;
      if (active && e >= 0 && e < E && q >= 0 && q < L) key = q;
    }
    keys[i] = key;
  }
  for (int i = tid; i < L; i += blockDim.x) carry[i] = 0;
#pragma unroll
  for (int step = 0; step < kMaxSteps; ++step) {
    const int f0 = step * (int)blockDim.x;
    if (f0 >= n_routes) break;
    for (int i = tid; i < nw * L; i += blockDim.x) wave_cnt[i] = 0;
    const int f = f0 + tid;
    const int key = keys[step];
    uint64_t same = __ballot(1);
    for (int b = 0; b < nbits; ++b) {
      const int bit = (key >> b) & 1;
      const uint64_t bal = __ballot(bit);
      same &= bit ? bal : ~bal;
    }
    const int rank_in_wave = __popcll(same & lanes_below(lane));
    __syncthreads();
    if (key < L && rank_in_wave == 0) wave_cnt[wv * L + key] = __popcll(same);
    __syncthreads();
    for (int le = tid; le < L; le += blockDim.x) {
      int run = carry[le];
      for (int w = 0; w < nw; ++w) {
        const int v = wave_cnt[w * L + le];
        wave_cnt[w * L + le] = run;
        run += v;
      }
      carry[le] = run;
    }
    __syncthreads();
    if (f < n_routes) {
      P[f_base + f] = (key < L) ? (key | ((wave_cnt[wv * L + key] + rank_in_wave) << 16)) : -1;
    }
    __syncthreads();
  }
  for (int le = tid; le < L; le += blockDim.x) cnt[counter_slot((le * W + s) * G + g)] = carry[le];
}

// ---------------------------------------------------------------------------
// a2 inside one wavefront: exclusive scan of the group counters in
// (le, s, g) order, kScanIPL consecutive counters per lane per chunk.  The
// exclusive prefix at (le, s, g) is the first row of that group's routes to
// le; the inclusive prefix at the last group of (le, s) is
// epRecvCounts[le*W + s] ([TL] GetCumSum and local data copy: receive count
// = begin + count).  Returns the exclusive prefix at q (lanes with q < 0 get
// 0).  With `writer`, also stores epRecvCounts.  `first` holds this lane's
// counters of chunk 0, loaded early by the caller.
// ---------------------------------------------------------------------------

__device__ __forceinline__ void load_counters(const int32_t* __restrict__ cnt, int n, int c0, int lane,
                                              int (&v)[kScanIPL]) {
  const int i0 = c0 + lane * kScanIPL;
#pragma unroll
  for (int j = 0; j < kScanIPL; ++j) v[j] = (i0 + j < n) ? cnt[c0 + j * 64 + lane] : 0;
}

// Orders this wavefront's LDS accesses: the LDS work issued so far completes
// before anything after it is issued.
__device__ __forceinline__ void lds_wave_sync() {
  __builtin_amdgcn_s_waitcnt(0xC07F);  // lgkmcnt(0), vmcnt/expcnt untouched
  __builtin_amdgcn_wave_barrier();
}

__device__ int scan_lookup(const int32_t* __restrict__ cnt, int n, const int (&first)[kScanIPL], int q, int G,
                           bool writer, int32_t* __restrict__ ep_recv, int lane, int32_t* __restrict__ pref) {
  int carry = 0;
  int found = 0;
  for (int c0 = 0; c0 < n; c0 += kScanChunk) {
    int v[kScanIPL];
    if (c0 == 0) {
#pragma unroll
      for (int j = 0; j < kScanIPL; ++j) v[j] = first[j];
    } else {
      load_counters(cnt, n, c0, lane, v);
    }
    int ex[kScanIPL];
    int sum = 0;
#pragma unroll
    for (int j = 0; j < kScanIPL; ++j) {
      ex[j] = sum;
      sum += v[j];
    }
    const int incl = wave_inclusive_scan(sum);
    const int lane_base = carry + incl - sum;
    const int i0 = c0 + lane * kScanIPL;
#pragma unroll
    for (int j = 0; j < kScanIPL; ++j) pref[lane * kScanIPL + j] = lane_base + ex[j];
    if (writer) {
#pragma unroll
      for (int j = 0; j < kScanIPL; ++j) {
        const int i = i0 + j;
        if (i < n && (i % G) == G - 1) ep_recv[i / G] = lane_base + ex[j] + v[j];
      }
    }
    lds_wave_sync();
    const int rel = q - c0;
    if (q >= 0 && rel >= 0 && rel < kScanChunk) found = pref[rel];
    carry += __builtin_amdgcn_readlane(incl, 63);
    lds_wave_sync();
  }
  return found;
}

// ---------------------------------------------------------------------------
// a2 + a3 (rows) + a4 + a5: one wavefront per (source token, column tile).
// Lanes 0..K-1 read the token's ranks; if any route is sent to this rank the
// wavefront loads its column tile of x[s][t] once, turns ranks into rows
// (group base from the in-wavefront scan + rank), and writes the tile to each
// of the token's rows with non-temporal stores ([TL] send loop row put and
// local data copy; [PTO] Dispatch Stage: destination rows grouped by local
// expert then source).  Rows at or beyond the capacity A are dropped.  Tile 0
// writes the (s, t, k) triplets and the inverse index; the wavefront of token
// 0, tile 0 also writes epRecvCounts and expertTokenNums
// ([TL] UpdateTokenNumsOut: per-local-expert counts).
// ---------------------------------------------------------------------------
template <int VPL>
__global__ __launch_bounds__(64 * MDC_GATHER_WAVES) void k_dispatch_gather(
    const v4u* __restrict__ x, const int32_t* __restrict__ P, const int32_t* __restrict__ cnt,
    v4u* __restrict__ expand_x, int32_t* __restrict__ assist, int32_t* __restrict__ ep_recv,
    int64_t* __restrict__ expert_nums, int32_t* __restrict__ row_idx,
    int BS, int K, int L, int W, int TPG, int G, int64_t A, int nvec, int ntiles, unsigned n_items) {
  const unsigned item = blockIdx.x * MDC_GATHER_WAVES + (threadIdx.x >> 6);
  if (item >= n_items) return;
  const unsigned gu = item / (unsigned)ntiles;
  const int tile = (int)(item - gu * (unsigned)ntiles);
  const int s = (int)(gu / (unsigned)BS);
  const int t = (int)(gu - (unsigned)s * (unsigned)BS);
  const int64_t g = gu;
  const int lane = threadIdx.x & 63;

  const bool writer = (g == 0) && (tile == 0);
  const int n_cnt = L * W * G;
  int cnt0[kScanIPL];
  load_counters(cnt, n_cnt, 0, lane, cnt0);
  const int p = (lane < K) ? P[g * K + lane] : -1;
  const bool mine = (p >= 0) && ((p & 0xFFFF) < L);
  const uint64_t has = __ballot(mine);
  if (has == 0 && !writer) return;

  // Column tile of the source row: issued before the scan so the loads overlap it.
  const int base = tile * 64 * VPL + lane;
  const bool full = (tile + 1) * 64 * VPL <= nvec;
  const uint64_t src = (uint64_t)(x + g * nvec);
  v4u v[VPL];
  if (has != 0) {
    if (full) {
#pragma unroll
      for (int u = 0; u < VPL; ++u) v[u] = load_v4<MDC_GATHER_NT_LOADS != 0>(src + (uint64_t)(base + u * 64) * 16);
    } else {
#pragma unroll
      for (int u = 0; u < VPL; ++u) {
        const int idx = base + u * 64;
        v[u] = idx < nvec ? load_v4<MDC_GATHER_NT_LOADS != 0>(src + (uint64_t)idx * 16) : v4u{0u, 0u, 0u, 0u};
      }
    }
  }

  const int le = p & 0xFFFF;
  const int q = mine ? ((le * W + s) * G + t / TPG) : -1;
  __shared__ int32_t pref_all[MDC_GATHER_WAVES][kScanChunk];
  const int first = scan_lookup(cnt, n_cnt, cnt0, q, G, writer, ep_recv, lane, pref_all[threadIdx.x >> 6]);
  if (writer) {
    for (int e = lane; e < L; e += 64) {
      int64_t sum = 0;
      for (int i = 0; i < W * G; ++i) sum += cnt[counter_slot(e * W * G + i)];
      expert_nums[e] = sum;
    }
  }
  if (has == 0) return;

  int row = -1;
  if (mine) {
    const int64_t r = (int64_t)first + (p >> 16);
    row = (r >= 0 && r < A) ? (int)r : -1;
  }
  if (tile == 0 && mine) {
    row_idx[g * K + lane] = row;
    if (row >= 0) {
      int32_t* a = assist + (int64_t)row * 3;
      a[0] = s;
      a[1] = t;
      a[2] = lane;
    }
  }
  uint64_t rem = __ballot(row >= 0);
  while (rem) {
    const int k = __ffsll((unsigned long long)rem) - 1;
    rem &= rem - 1;
    const int rk = __builtin_amdgcn_readlane(row, k);
    v4u* dst = expand_x + (int64_t)rk * nvec;
    if (full) {
#pragma unroll
      for (int u = 0; u < VPL; ++u) store_v4<MDC_GATHER_NT_STORES != 0>(dst + base + u * 64, v[u]);
    } else {
#pragma unroll
      for (int u = 0; u < VPL; ++u) {
        const int idx = base + u * 64;
        if (idx < nvec) store_v4<MDC_GATHER_NT_STORES != 0>(dst + idx, v[u]);
      }
    }
  }
}

// ---------------------------------------------------------------------------
// Quantised dispatch ([CV4] int8 communication quantisation; [PTO]
// FrontReorder Stage: quantised token rows with a per-token scale): one
// wavefront per source token with a local route reads the whole row once,
// quantises it per row in fp32 (amax / 127, round half even, clamp +-127) and
// writes the int8 row and its scale to each destination row.  Placement,
// triplets, inverse index and counts are those of k_dispatch_gather.
// Rows of up to 64 * 16 vectors (H <= 8192) are held in registers.
// ---------------------------------------------------------------------------
constexpr int kQuantRowVec = 16;

template <int VPL>
__global__ __launch_bounds__(64) void k_dispatch_gather_q(
    const v4u* __restrict__ x, const int32_t* __restrict__ P, const int32_t* __restrict__ cnt,
    int8_t* __restrict__ expand_q, float* __restrict__ dyn_scale, int32_t* __restrict__ assist,
    int32_t* __restrict__ ep_recv, int64_t* __restrict__ expert_nums, int32_t* __restrict__ row_idx,
    int BS, int K, int L, int W, int TPG, int G, int64_t A, int nvec) {
  const unsigned gu = blockIdx.x;
  const int s = (int)(gu / (unsigned)BS);
  const int t = (int)(gu - (unsigned)s * (unsigned)BS);
  const int64_t g = gu;
  const int lane = threadIdx.x & 63;
  const bool writer = (g == 0);
  const int n_cnt = L * W * G;
  int cnt0[kScanIPL];
  load_counters(cnt, n_cnt, 0, lane, cnt0);
  const int p = (lane < K) ? P[g * K + lane] : -1;
  const bool mine = (p >= 0) && ((p & 0xFFFF) < L);
  const uint64_t has = __ballot(mine);
  if (has == 0 && !writer) return;

  const uint64_t src = (uint64_t)(x + g * nvec);
  v4u v[VPL];
  if (has != 0) {
#pragma unroll
    for (int u = 0; u < VPL; ++u) {
      const int idx = lane + u * 64;
      v[u] = idx < nvec ? load_v4<MDC_GATHER_NT_LOADS != 0>(src + (uint64_t)idx * 16) : v4u{0u, 0u, 0u, 0u};
    }
  }
  const int le = p & 0xFFFF;
  const int q = mine ? ((le * W + s) * G + t / TPG) : -1;
  __shared__ int32_t pref_all[kScanChunk];
  const int first = scan_lookup(cnt, n_cnt, cnt0, q, G, writer, ep_recv, lane, pref_all);
  if (writer) {
    for (int e = lane; e < L; e += 64) {
      int64_t sum = 0;
      for (int i = 0; i < W * G; ++i) sum += cnt[counter_slot(e * W * G + i)];
      expert_nums[e] = sum;
    }
  }
  if (has == 0) return;

  // per-row quantisation, decided in fp32
  float amax = 0.f;
#pragma unroll
  for (int u = 0; u < VPL; ++u)
#pragma unroll
    for (int w = 0; w < 4; ++w) amax = fmaxf(amax, fmaxf(fabsf(bf16_lo(v[u][w])), fabsf(bf16_hi(v[u][w]))));
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) amax = fmaxf(amax, __shfl_xor(amax, o, 64));
  const float inv = amax > 0.f ? 127.0f / amax : 0.f;
  const float scale = amax / 127.0f;
  uint64_t qv[VPL];
#pragma unroll
  for (int u = 0; u < VPL; ++u) {
    uint64_t packed = 0;
#pragma unroll
    for (int w = 0; w < 4; ++w) {
      const float a = fminf(fmaxf(rintf(bf16_lo(v[u][w]) * inv), -127.f), 127.f);
      const float b = fminf(fmaxf(rintf(bf16_hi(v[u][w]) * inv), -127.f), 127.f);
      packed |= (uint64_t)(uint8_t)(int8_t)(int)a << (16 * w);
      packed |= (uint64_t)(uint8_t)(int8_t)(int)b << (16 * w + 8);
    }
    qv[u] = packed;
  }

  int row = -1;
  if (mine) {
    const int64_t r = (int64_t)first + (p >> 16);
    row = (r >= 0 && r < A) ? (int)r : -1;
  }
  if (mine) {
    row_idx[g * K + lane] = row;
    if (row >= 0) {
      int32_t* a = assist + (int64_t)row * 3;
      a[0] = s;
      a[1] = t;
      a[2] = lane;
      dyn_scale[row] = scale;
    }
  }
  uint64_t rem = __ballot(row >= 0);
  while (rem) {
    const int k = __ffsll((unsigned long long)rem) - 1;
    rem &= rem - 1;
    const int rk = __builtin_amdgcn_readlane(row, k);
    uint64_t* dst = reinterpret_cast<uint64_t*>(expand_q + (int64_t)rk * nvec * 8);
#pragma unroll
    for (int u = 0; u < VPL; ++u) {
      const int idx = lane + u * 64;
      if (idx < nvec) {
        if (MDC_GATHER_NT_STORES) __builtin_nontemporal_store(qv[u], dst + idx);
        else dst[idx] = qv[u];
      }
    }
  }
}

// Empty batch: every count is zero.
__global__ __launch_bounds__(64) void k_zero_counts(int32_t* __restrict__ ep_recv, int64_t* __restrict__ expert_nums,
                                                    int L, int W) {
  for (int i = threadIdx.x; i < L * W; i += 64) ep_recv[i] = 0;
  for (int i = threadIdx.x; i < L; i += 64) expert_nums[i] = 0;
}

// ---------------------------------------------------------------------------
// a6: combine.  One wavefront per (token t of rank r, column tile).
// ---------------------------------------------------------------------------
struct CombineTables {
  const v4u* y[MDC_MAX_COMBINE_WORLD];
  const int32_t* assist[MDC_MAX_COMBINE_WORLD];
  const int32_t* counts[MDC_MAX_COMBINE_WORLD];
};


// Route (r, t, k) is present when the token is active, 0 <= e < E, and row
// idx[t][k] of destination j = e / L is below min(count_j, A) and holds the
// triplet (r, t, k).  The prologue is two load levels: (ids, row index,
// scale, mask, pointer tables) then (count_j, triplet); every address is
// kept inside its buffer so the loads can be issued without branches.
template <int KMAX, int V, bool SHARED>
__global__ __launch_bounds__(64 * MDC_COMBINE_WAVES) void k_combine(
    CombineTables tabs, const int32_t* __restrict__ row_idx, const int32_t* __restrict__ ids,
    const float* __restrict__ scales, const uint8_t* __restrict__ mask,
    const v4u* __restrict__ shared, const v4u* __restrict__ ori, v4u* __restrict__ out,
    int r, int W, int K, int E, int L, int64_t A, int nvec, int ntiles, unsigned n_items,
    int mask_per_route, int Z, int C) {
  const unsigned item = blockIdx.x * MDC_COMBINE_WAVES + (threadIdx.x >> 6);
  if (item >= n_items) return;
  const int t = (int)(item / (unsigned)ntiles);
  const int tile = (int)(item - (unsigned)t * (unsigned)ntiles);
  const int lane = threadIdx.x & 63;
  const int kk = lane < K ? lane : 0;
  const int64_t rt = (int64_t)t * K + kk;

  const int e = ids[rt];
  const int row = row_idx[rt];
  const float sc = scales[rt];
  const bool act = (mask == nullptr) || (mask[mask_per_route ? rt : (int64_t)t] != 0);
  const int tl = lane < W ? lane : 0;
  const uint64_t yb = (uint64_t)tabs.y[tl];
  const uint64_t ab = (uint64_t)tabs.assist[tl];
  const uint64_t cb = (uint64_t)tabs.counts[tl];

  const bool valid = (lane < K) && act && e >= 0 && e < E && A > 0;
  const int j = valid ? e / L : 0;
  const bool inrange = row >= 0 && row < A;
  const int64_t rowc = inrange ? row : 0;
  const uint64_t yj = shfl64(yb, j);
  const uint64_t aj = shfl64(ab, j);
  const uint64_t cj = shfl64(cb, j);

  bool ok = false;
  if (A > 0) {
    const int32_t total = load_i32(cj + ((uint64_t)L * W - 1) * 4);
    const uint64_t a = aj + (uint64_t)rowc * 12;
    const int a0 = load_i32(a), a1 = load_i32(a + 4), a2 = load_i32(a + 8);
    ok = valid && inrange && row < total && a0 == r && a1 == t && a2 == lane;
  }
  v4u* orow = out + (int64_t)t * nvec;
  // Zero experts [E, E+Z) and copy experts [E+Z, E+Z+C) are present without a
  // dispatched row: output 0 (read from a valid row, then replaced by zero) or
  // the token's own row ori[t].
  const bool special = (lane < K) && act && e >= E && e - E < Z + C;
  const bool is_zero = special && e - E < Z;
  uint64_t yrow = yj + (uint64_t)rowc * (uint64_t)nvec * sizeof(v4u);
  if (special) yrow = is_zero ? (uint64_t)orow : (uint64_t)(ori + (int64_t)t * nvec);
  ok = ok || special;
  const uint64_t has = __ballot(ok);
  const uint64_t zero_lanes = __ballot(is_zero);
  const int np = __popcll(has);
  const int base = tile * 64 * V + lane;

  if (np == 0) {
    const v4u z = {0u, 0u, 0u, 0u};
#pragma unroll
    for (int u = 0; u < V; ++u) {
      const int idx = base + u * 64;
      if (idx < nvec) store_v4<MDC_COMBINE_NT_STORES != 0>(orow + idx, z);
    }
    return;
  }

  // Present routes in ascending k as wavefront-uniform row addresses and scales;
  // slots past the last present route repeat the first one (loaded, never summed).
  uint64_t yp[KMAX];
  float sk[KMAX];
  bool zk[KMAX];
  uint64_t rem = has;
#pragma unroll
  for (int i = 0; i < KMAX; ++i) {
    const int k = rem ? (__ffsll((unsigned long long)rem) - 1) : (__ffsll((unsigned long long)has) - 1);
    yp[i] = readlane64(yrow, k);
    sk[i] = __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, sc), k));
    zk[i] = (zero_lanes >> k) & 1;
    rem &= rem - 1;
  }

  v4u yv[KMAX][V];
  v4u shv[V];
  const uint64_t srow = (uint64_t)(shared + (int64_t)t * nvec);
  const bool full = (tile + 1) * 64 * V <= nvec;
  if (full) {
#pragma unroll
    for (int i = 0; i < KMAX; ++i)
#pragma unroll
      for (int u = 0; u < V; ++u) yv[i][u] = load_v4<MDC_COMBINE_NT_LOADS != 0>(yp[i] + (uint64_t)(base + u * 64) * sizeof(v4u));
    if (SHARED) {
#pragma unroll
      for (int u = 0; u < V; ++u) shv[u] = load_v4<MDC_COMBINE_NT_LOADS != 0>(srow + (uint64_t)(base + u * 64) * sizeof(v4u));
    }
  } else {
#pragma unroll
    for (int i = 0; i < KMAX; ++i)
#pragma unroll
      for (int u = 0; u < V; ++u) {
        const int idx = base + u * 64;
        yv[i][u] = (idx < nvec) ? load_v4<MDC_COMBINE_NT_LOADS != 0>(yp[i] + (uint64_t)idx * sizeof(v4u)) : v4u{0u, 0u, 0u, 0u};
      }
    if (SHARED) {
#pragma unroll
      for (int u = 0; u < V; ++u) {
        const int idx = base + u * 64;
        shv[u] = (idx < nvec) ? load_v4<MDC_COMBINE_NT_LOADS != 0>(srow + (uint64_t)idx * sizeof(v4u)) : v4u{0u, 0u, 0u, 0u};
      }
    }
  }
#pragma unroll
  for (int i = 0; i < KMAX; ++i)
#pragma unroll
    for (int u = 0; u < V; ++u)
      if (zk[i]) yv[i][u] = v4u{0u, 0u, 0u, 0u};
#pragma unroll
  for (int u = 0; u < V; ++u) {
    const int idx = base + u * 64;
    float acc[8];
#pragma unroll
    for (int c = 0; c < 8; ++c) acc[c] = 0.f;
#pragma unroll
    for (int i = 0; i < KMAX; ++i) {
      if (i < np) {
        const float s_ = sk[i];
#pragma unroll
        for (int w = 0; w < 4; ++w) {
          const unsigned yw = yv[i][u][w];
          const float a0 = s_ * bf16_lo(yw);
          const float a1 = s_ * bf16_hi(yw);
          if (SHARED) {
            const unsigned sw = shv[u][w];
            const float b0 = s_ * bf16_lo(sw);
            const float b1 = s_ * bf16_hi(sw);
            acc[2 * w] = acc[2 * w] + (a0 + b0);
            acc[2 * w + 1] = acc[2 * w + 1] + (a1 + b1);
          } else {
            acc[2 * w] = acc[2 * w] + a0;
            acc[2 * w + 1] = acc[2 * w + 1] + a1;
          }
        }
      }
    }
    v4u o;
#pragma unroll
    for (int w = 0; w < 4; ++w) o[w] = bf16_rne(acc[2 * w]) | (bf16_rne(acc[2 * w + 1]) << 16);
    if (idx < nvec) store_v4<MDC_COMBINE_NT_STORES != 0>(orow + idx, o);
  }
}

// ---------------------------------------------------------------------------
// a7: grouped int8 expert FFN ([PTO] GMM1 / SwiGLU / GMM2 stages).
//
// Per local expert e, on its expert-major rows of expand_x:
//   q1, s1 = per-row int8 quantisation of x (amax / 127, round half even)
//   h      = (q1 . W1[e]^T) * s1[row] * w1s[e][n]          (int32 MFMA accumulate)
//   g      = silu(h[:, j]) * h[:, j + N/2],  j < N/2        (fused in GMM1's epilogue)
//   q2, s2 = per-row int8 quantisation of g (quantised while GMM2 loads its tiles)
//   y      = bf16((q2 . W2[e]^T) * s2[row] * w2s[e][h])
// The GEMMs use v_mfma_i32_32x32x32_i8 on 256-token x 256-weight-row tiles
// (GMM1: 128 gate + 128 up weight rows per tile so gate and up land in the
// same lanes), eight wavefronts (two per SIMD) each holding a 128 x 64 int32
// accumulator block in AGPRs, k staged through a double-buffered LDS ring 128
// bytes deep; the output tile leaves through LDS as whole rows.
// ---------------------------------------------------------------------------
typedef int v4i __attribute__((ext_vector_type(4)));
typedef int v16i __attribute__((ext_vector_type(16)));

constexpr int kFfnBM = 256;        // token rows per tile
constexpr int kFfnBW = 256;        // weight rows per tile (GMM1: 128 gate + 128 up)
constexpr int kFfnBK = 128;        // k bytes per LDS stage
constexpr int kFfnThreads = 512;   // 8 wavefronts: 2 along tokens x 4 along weight rows
constexpr int kFfnStage = (kFfnBM + kFfnBW) * kFfnBK;   // bytes of one LDS stage
constexpr int kFfnOutAlign = 128;  // GMM output widths (N/2 and H) must be multiples of this

// Tile plan shared by both GEMMs.  Each local expert's rows (contiguous,
// expert-major, clipped at A) split into m-tiles of kFfnBM rows.  The table
// lists every full m-tile first (expert order), then each expert's partial
// last m-tile by row count, largest first: the persistent GEMMs walk tiles
// in table order, so the workgroups that run one tile more than the others
// end on the cheapest tiles.  tiles[0].x = number of m-tiles; tiles[1 + m] =
// {expert, first row, expert's end row, 0}.  One workgroup of 1024 threads;
// L <= 2048 (two experts per thread).
constexpr int kPlanThreads = 1024;

// Exclusive prefix over the 2048 values held two per thread (elements 2t and
// 2t + 1); returns the prefix of element 2t and the grand total.
__device__ int64_t plan_scan_pair(int64_t a, int64_t b, int64_t* wsum, int64_t& total) {
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int64_t own = a + b;
  int64_t s = own;
#pragma unroll
  for (int o = 1; o < 64; o <<= 1) {
    const int64_t n = __shfl_up(s, o, 64);
    if (lane >= o) s += n;
  }
  if (lane == 63) wsum[wave] = s;
  __syncthreads();
  if (tid == 0) {
    int64_t run = 0;
    for (int w = 0; w < kPlanThreads / 64; ++w) {
      const int64_t x = wsum[w];
      wsum[w] = run;
      run += x;
    }
    wsum[kPlanThreads / 64] = run;
  }
  __syncthreads();
  const int64_t excl = wsum[wave] + s - own;
  total = wsum[kPlanThreads / 64];
  __syncthreads();   // wsum is reused by the next scan
  return excl;
}

__global__ __launch_bounds__(kPlanThreads) void k_ffn_plan(const int64_t* __restrict__ expert_nums, int L, int64_t A,
                                                           int4* __restrict__ tiles) {
  __shared__ int rem_s[2 * kPlanThreads];
  __shared__ int64_t wsum[kPlanThreads / 64 + 1];
  const int tid = threadIdx.x;
  const int e0 = 2 * tid, e1 = 2 * tid + 1;
  const int64_t c0 = e0 < L ? expert_nums[e0] : 0, c1 = e1 < L ? expert_nums[e1] : 0;
  int64_t total;
  const int64_t x0 = plan_scan_pair(c0, c1, wsum, total);   // first row of e0 (unclipped)
  const int64_t x1 = x0 + c0;
  const int lo0 = (int)min(x0, A), hi0 = (int)min(x0 + c0, A);
  const int lo1 = (int)min(x1, A), hi1 = (int)min(x1 + c1, A);
  const int f0 = (hi0 - lo0) / kFfnBM, f1 = (hi1 - lo1) / kFfnBM;   // full m-tiles
  const int r0 = (hi0 - lo0) % kFfnBM, r1 = (hi1 - lo1) % kFfnBM;   // rows of the partial m-tile
  rem_s[e0] = r0;
  rem_s[e1] = r1;
  int64_t nfull;
  const int fp0 = (int)plan_scan_pair(f0, f1, wsum, nfull);          // table slot of e0's first full tile
  int64_t npart;
  (void)plan_scan_pair(r0 > 0, r1 > 0, wsum, npart);                // also orders rem_s writes before reads
  for (int f = 0; f < f0; ++f) tiles[1 + fp0 + f] = int4{e0, lo0 + f * kFfnBM, hi0, 0};
  for (int f = 0; f < f1; ++f) tiles[1 + fp0 + f0 + f] = int4{e1, lo1 + f * kFfnBM, hi1, 0};
  // partial tiles: rank by rows, descending, ties by expert
  for (int h = 0; h < 2; ++h) {
    const int e = h ? e1 : e0, r = h ? r1 : r0;
    if (e >= L || r == 0) continue;
    int rank = 0;
    for (int o = 0; o < L; ++o) {
      const int ro = rem_s[o];
      rank += (ro > r) || (ro == r && o < e);
    }
    const int lo = h ? lo1 : lo0, f = h ? f1 : f0, hi = h ? hi1 : hi0;
    tiles[1 + (int)nfull + rank] = int4{e, lo + f * kFfnBM, hi, 0};
  }
  if (tid == 0) tiles[0] = int4{(int)(nfull + npart), 0, 0, 0};
}

__device__ __forceinline__ float ffn_silu(float a) { return a * __builtin_amdgcn_rcpf(1.0f + __expf(-a)); }

// Two fp32 -> two bf16 (round to nearest even, one v_cvt_pk_bf16_f32), lo in
// the low half.
typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
typedef float f32x2_t __attribute__((ext_vector_type(2)));
__device__ __forceinline__ uint32_t ffn_pack_bf16(float lo, float hi) {
  return __builtin_bit_cast(uint32_t, __builtin_convertvector((f32x2_t){lo, hi}, bf16x2_t));
}

// Per-row int8 quantisation of bf16 rows of `width` elements, decided in fp32
// exactly as: amax = max|v|, inv = 127 / amax, q = clamp(rint(v * inv), -127,
// 127), scale = amax / 127 (a zero row gives q = 0, scale = 0).  One
// wavefront per row, rows [0, min(sum(expert_nums), A)) visited grid-stride;
// rows of up to 64 * kQuantVec vectors stay in registers between the passes.
constexpr int kQuantVec = 16;
__global__ __launch_bounds__(256) void k_ffn_quant_rows(
    const v4u* __restrict__ x, int8_t* __restrict__ q, float* __restrict__ scale,
    const int64_t* __restrict__ expert_nums, int L, int64_t A, int nvec) {
  const int lane = threadIdx.x & 63;
  const int64_t nw = (int64_t)gridDim.x * 4;
  int64_t total = 0;
  for (int i = 0; i < L; ++i) total += expert_nums[i];
  const int64_t rows = total < A ? total : A;
  for (int64_t row = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6); row < rows; row += nw) {
    const v4u* xr = x + row * nvec;
    uint64_t* qr = reinterpret_cast<uint64_t*>(q + row * (int64_t)nvec * 8);
    v4u cache[kQuantVec];
    float amax = 0.f;
    if (nvec <= 64 * kQuantVec) {
#pragma unroll
      for (int u = 0; u < kQuantVec; ++u) {
        const int i = lane + 64 * u;
        cache[u] = i < nvec ? xr[i] : v4u{0u, 0u, 0u, 0u};
      }
#pragma unroll
      for (int u = 0; u < kQuantVec; ++u)
#pragma unroll
        for (int w = 0; w < 4; ++w)
          amax = fmaxf(amax, fmaxf(fabsf(bf16_lo(cache[u][w])), fabsf(bf16_hi(cache[u][w]))));
    } else {
      for (int i = lane; i < nvec; i += 64) {
        const v4u v = xr[i];
#pragma unroll
        for (int w = 0; w < 4; ++w) amax = fmaxf(amax, fmaxf(fabsf(bf16_lo(v[w])), fabsf(bf16_hi(v[w]))));
      }
    }
#pragma unroll
    for (int o = 32; o >= 1; o >>= 1) amax = fmaxf(amax, __shfl_xor(amax, o, 64));
    const float inv = amax > 0.f ? 127.0f / amax : 0.f;
    auto quant8 = [&](const v4u& v) {
      uint64_t packed = 0;
#pragma unroll
      for (int w = 0; w < 4; ++w) {
        const float a = fminf(fmaxf(rintf(bf16_lo(v[w]) * inv), -127.f), 127.f);
        const float b = fminf(fmaxf(rintf(bf16_hi(v[w]) * inv), -127.f), 127.f);
        packed |= (uint64_t)(uint8_t)(int8_t)(int)a << (16 * w);
        packed |= (uint64_t)(uint8_t)(int8_t)(int)b << (16 * w + 8);
      }
      return packed;
    };
    if (nvec <= 64 * kQuantVec) {
#pragma unroll
      for (int u = 0; u < kQuantVec; ++u) {
        const int i = lane + 64 * u;
        if (i < nvec) qr[i] = quant8(cache[u]);
      }
    } else {
      for (int i = lane; i < nvec; i += 64) qr[i] = quant8(xr[i]);
    }
    if (lane == 0) scale[row] = amax / 127.0f;
  }
}

// The k loop of one tile (see k_ffn_gemm).  Stage ks + 1 travels global ->
// registers during stage ks - 1 and registers -> LDS during stage ks, into the
// buffer nobody reads in stage ks; one barrier ends each stage.  Fragments of
// k substep q + 1 are read while the MFMAs of substep q run, and the last
// substep's MFMAs run after the stage barrier, beside the next stage's first
// fragment reads.  Scheduling groups (sched_group_barrier masks: 0x8 MFMA,
// 0x100 LDS read, 0x200 LDS write, 0x20 global read) interleave the memory
// instructions with the MFMAs.
struct FfnStaging {
  __amdgpu_buffer_rsrc_t ra, rw;   // token rows, weight rows (range-checked)
  unsigned va, vw;                 // lane offsets of this thread's i = 0 rows
  unsigned whi;                    // extra weight offset of rows i >= 2 (GMM1: gate -> up)
  int K;
  int lds_off;                     // this thread's LDS byte offset for i = 0
};

// NB = number of the wavefront's 32-row token blocks that hold valid rows:
// blocks past them stay zero, and their fragment reads and MFMAs are not
// issued (an expert's short last m-tile is cheap).  NB = 0 still stages and
// joins the barriers.
template <bool GLU, int NB>
__device__ __forceinline__ void ffn_kloop(uint8_t* lds, v16i (&acc)[2][4], const FfnStaging& st, int wt, int wn,
                                          const int (&fr)[4]) {
  constexpr int NCOLS = GLU ? kFfnBW / 2 : kFfnBW;
  constexpr int NR = NB > 0 ? NB + 2 : 0;   // fragment reads per k substep
  constexpr int NM = 2 * NB;                // MFMAs per k substep
  // LDS row of weight block j (32 rows) within the stage's weight tile
  auto wrow = [&](int j) {
    if (GLU) return j == 0 ? wn * 32 : NCOLS + wn * 32;
    return wn * 64 + 32 * j;
  };
  v4i sa[4], sw[4];
  auto gload = [&](int k0) {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      sa[i] = __builtin_amdgcn_raw_buffer_load_b128(st.ra, st.va + (unsigned)(64 * i * st.K), (unsigned)k0, 0);
      sw[i] = __builtin_amdgcn_raw_buffer_load_b128(st.rw, st.vw + (unsigned)(64 * i * st.K) + (i >= 2 ? st.whi : 0u),
                                                    (unsigned)k0, 0);
    }
  };
  auto lwrite = [&](uint8_t* buf) {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      *reinterpret_cast<v4i*>(buf + st.lds_off + 64 * i * kFfnBK) = sa[i];
      *reinterpret_cast<v4i*>(buf + kFfnBM * kFfnBK + st.lds_off + 64 * i * kFfnBK) = sw[i];
    }
  };
  auto frags = [&](const uint8_t* sb, int q, v4i (&tf)[4], v4i (&wf)[2]) {
    if (NB == 0) return;
#pragma unroll
    for (int i = 0; i < NB; ++i) tf[i] = *reinterpret_cast<const v4i*>(sb + (wt * 128 + 32 * i) * kFfnBK + fr[q]);
#pragma unroll
    for (int j = 0; j < 2; ++j)
      wf[j] = *reinterpret_cast<const v4i*>(sb + kFfnBM * kFfnBK + wrow(j) * kFfnBK + fr[q]);
  };
  auto mfmas = [&](const v4i (&tf)[4], const v4i (&wf)[2]) {
#pragma unroll
    for (int i = 0; i < NB; ++i)
#pragma unroll
      for (int j = 0; j < 2; ++j) acc[j][i] = __builtin_amdgcn_mfma_i32_32x32x32_i8(wf[j], tf[i], acc[j][i], 0, 0, 0);
  };
  auto interleave_reads = [&]() {
#pragma unroll
    for (int n = 0; n < NR; ++n) {
      if (n < NM) __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
      __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
    }
    if (NM > NR) __builtin_amdgcn_sched_group_barrier(0x008, NM - NR, 0);
    __builtin_amdgcn_sched_barrier(0);
  };
  auto interleave_staging = [&]() {
#pragma unroll
    for (int n = 0; n < 8; ++n) {
      if (n < NM) __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
      if (n < 8) __builtin_amdgcn_sched_group_barrier(0x200, 1, 0);
      if (n < 8) __builtin_amdgcn_sched_group_barrier(0x020, 1, 0);
      if (n < NR) __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
    }
    __builtin_amdgcn_sched_barrier(0);
  };

  const int nk = st.K / kFfnBK;
  v4i tf[4], wf[2], tg[4], wg[2];
  gload(0);
  lwrite(lds);
  __syncthreads();
  gload(min(1, nk - 1) * kFfnBK);
  frags(lds, 0, tf, wf);
  for (int ks = 0; ks < nk; ++ks) {
    uint8_t* cur = lds + (ks & 1) * kFfnStage;
    uint8_t* nxt = lds + ((ks + 1) & 1) * kFfnStage;
    frags(cur, 1, tg, wg);
    mfmas(tf, wf);
    interleave_reads();
    // stage ks + 1: registers -> LDS, then stage ks + 2: global -> registers
    // (the last iterations repeat the last stage; nobody reads it)
    lwrite(nxt);
    gload(min(ks + 2, nk - 1) * kFfnBK);
    frags(cur, 2, tf, wf);
    mfmas(tg, wg);
    interleave_staging();
    frags(cur, 3, tg, wg);
    mfmas(tf, wf);
    interleave_reads();
    __syncthreads();
    frags(nxt, 0, tf, wf);
    mfmas(tg, wg);
    interleave_reads();
  }
}

// Persistent grouped GEMM, C = A . W[e]^T with A int8 [rows][K] (token rows
// of expert e) and W int8 [L][Nw][K].  GLU = true (GMM1): each tile pairs 128
// gate rows of W (columns n) with the 128 up rows (columns N/2 + n); the
// epilogue dequantises both, applies silu(gate) * up and writes bf16 g.
// GLU = false (GMM2): the epilogue dequantises and writes bf16 y.  Dequant:
// acc * row_scale[row] * w_scale[e][col].
//
// MFMA v_mfma_i32_32x32x32_i8: lane l supplies row l % 32 and k bytes
// 16 (l / 32) .. +16 of each 32 x 32 operand block and receives
// C[8 (r / 4) + 4 (l / 32) + r % 4][l % 32], r < 16.  The weight block is the
// first operand and the token block the second, so each lane holds runs of 4
// consecutive output columns of one token.  (This MFMA also updates its
// accumulator in place, which the 16 x 16 shapes do not get from the
// compiler: they copy accumulators every step.)
//
// Wavefront wv = 4 wt + wn holds tokens 128 wt .. +128 of the tile and weight
// rows 32 wn .. +32 (GMM1: those gate rows and the matching up rows) or
// 64 wn .. +64 (GMM2).  Two wavefronts per SIMD (one per token half) keep the
// MFMAs busy while the other one waits on LDS.
//
// LDS: two stages, each [256 token rows][128 B] + [256 weight rows][128 B].
// The 16-byte chunk c of row r sits at chunk c ^ ((r / 2) & 7) of that row,
// so any 16 consecutive rows read at one chunk cover all 16 bank groups.
// Out-of-range rows (past the expert's rows or past Nw) read as zero through
// the buffer descriptors' range checks and are never stored.
//
// Epilogue, per token half: the wavefronts of that half write their bf16
// outputs into LDS rows (row pitch padded by 8 bytes so 32 rows written at
// one column fall in distinct banks), then all wavefronts store whole rows
// with 16-byte stores.
//
// Tiles: T = (m-tiles of the plan) x (output columns / tile columns).
// The launch holds one workgroup per CU; workgroup b walks tiles
// i*G + (b % 8)*(G/8) + b / 8.  Hardware places workgroup b on XCD b % 8, so
// each XCD walks a contiguous run of tiles; tiles are ordered in groups of 4
// m-tiles x 8 n-tiles (m fastest), so the tiles an XCD runs together share A
// and W tiles in its L2.
template <bool GLU>
__global__ __launch_bounds__(kFfnThreads) void k_ffn_gemm(
    const int8_t* __restrict__ a_src, const float* __restrict__ row_scale,
    const int8_t* __restrict__ w, const float* __restrict__ w_scale, uint16_t* __restrict__ out,
    const int4* __restrict__ tiles, int K, int Nw, int Nout) {
  __shared__ __attribute__((aligned(16))) uint8_t lds[2 * kFfnStage];
  __shared__ float sc_row[kFfnBM];   // row scales of the tile's token rows
  __shared__ float sc_col[kFfnBW];   // weight-row scales (GMM1: 128 gate, then 128 up)
  constexpr int NCOLS = GLU ? kFfnBW / 2 : kFfnBW;   // output columns per tile
  constexpr int OU = NCOLS / 8;                      // 16-byte output units per tile row
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  // wavefront-uniform values are read into scalar registers (readfirstlane)
  const int wv = __builtin_amdgcn_readfirstlane(tid >> 6);
  // SIMD s runs wavefronts s and s + 4: one of each token half
  const int wt = wv >> 2;   // token half of the tile
  const int wn = wv & 3;    // weight-row quarter of the tile
  const int G = gridDim.x;
  const int nn = (Nout + NCOLS - 1) / NCOLS;
  constexpr int GM = 4, GN = 8;
  const int MT = tiles[0].x;
  const int64_t T = (int64_t)MT * nn;
  const int b = blockIdx.x;
  const int lin = (b % 8) * (G / 8) + b / 8;   // XCD-contiguous walk (G is a multiple of 8)

  // staging: thread t moves chunk t & 7 of rows 64 i + t / 8 (i < 4) of both
  // tiles; in LDS that chunk sits at slot (t & 7) ^ ((row / 2) & 7), and
  // (row / 2) & 7 = (t / 16) & 7 for every i
  const int st_row = tid >> 3;
  const int st_chunk = tid & 7;
  const int st_lds = st_row * kFfnBK + ((st_chunk ^ ((tid >> 4) & 7)) << 4);
  // fragment reads: lane l reads row l & 31, chunk 2 s + l / 32 (k substep s)
  int fr[4];
#pragma unroll
  for (int q = 0; q < 4; ++q) fr[q] = (lane & 31) * kFfnBK + (((2 * q + (lane >> 5)) ^ ((lane >> 1) & 7)) << 4);

  for (int64_t t = lin; t < T; t += G) {
    // tile t -> (m-tile, n-tile): groups of GM m-tiles x GN n-tiles, m fastest
    const int64_t band = (int64_t)GM * nn;
    const int64_t mg = t / band;
    const int64_t r = t - mg * band;
    const int m_in_group = (int)min((int64_t)GM, (int64_t)MT - mg * GM);
    const int64_t per_ng = (int64_t)m_in_group * GN;
    const int64_t ng = r / per_ng;
    const int64_t r2 = r - ng * per_ng;
    const int n_in_group = (int)min((int64_t)GN, (int64_t)nn - ng * GN);
    const int mt = (int)(mg * GM + r2 % m_in_group);
    const int nt = (int)(ng * GN + (r2 / m_in_group) % n_in_group);
    __syncthreads();   // the previous tile's epilogue is done with LDS
    const int4 ti = tiles[1 + mt];
    const int e = __builtin_amdgcn_readfirstlane(ti.x);
    const int row0 = __builtin_amdgcn_readfirstlane(ti.y);
    const int row_end = __builtin_amdgcn_readfirstlane(ti.z);
    const int n0 = nt * NCOLS;

    // buffer descriptors: token rows [row0, min(row_end, row0 + 256)) and
    // weight rows [n0, Nw) of expert e (GMM1 up rows at Nw/2 + n0 + ...)
    const int rows_here = min(row_end - row0, kFfnBM);
    const __amdgpu_buffer_rsrc_t ra = __builtin_amdgcn_make_buffer_rsrc(
        const_cast<int8_t*>(a_src + (int64_t)row0 * K), (short)0, rows_here * K, 0x00020000);
    const __amdgpu_buffer_rsrc_t rw = __builtin_amdgcn_make_buffer_rsrc(
        const_cast<int8_t*>(w + ((int64_t)e * Nw + n0) * K), (short)0, (Nw - n0) * K, 0x00020000);
    // weight rows (relative to n0): i < 2 -> rows 64 i + t / 8 (GMM1: gate),
    // i >= 2 -> GMM1: up rows Nw/2 + 64 (i - 2) + t / 8, GMM2: rows 64 i + t / 8
    const unsigned whi = GLU ? (unsigned)((Nw / 2 - NCOLS) * K) : 0u;
    const unsigned v0 = (unsigned)(st_row * K + st_chunk * 16);
    const FfnStaging st{ra, rw, v0, v0, whi, K, st_lds};

    // the epilogue's scales, read from LDS after the k loop's first barrier
    if (tid < kFfnBM) {
      sc_row[tid] = row_scale[min(row0 + tid, row_end - 1)];
    } else {
      const int c = tid - kFfnBM;
      const int wr = GLU ? (c < NCOLS ? n0 + c : Nw / 2 + n0 + (c - NCOLS)) : min(n0 + c, Nw - 1);
      sc_col[c] = w_scale[(int64_t)e * Nw + wr];
    }

    // acc[j][i]: weight block j (32 rows), token block i (32 rows)
    v16i acc[2][4];
#pragma unroll
    for (int j = 0; j < 2; ++j)
#pragma unroll
      for (int i = 0; i < 4; ++i) acc[j][i] = v16i{};
    // 32-row token blocks of this wavefront's half that hold valid rows
    const int nblk = __builtin_amdgcn_readfirstlane(min(4, max(0, (rows_here - wt * 128 + 31) / 32)));
    switch (nblk) {
      case 4: ffn_kloop<GLU, 4>(lds, acc, st, wt, wn, fr); break;
      case 3: ffn_kloop<GLU, 3>(lds, acc, st, wt, wn, fr); break;
      case 2: ffn_kloop<GLU, 2>(lds, acc, st, wt, wn, fr); break;
      case 1: ffn_kloop<GLU, 1>(lds, acc, st, wt, wn, fr); break;
      default: ffn_kloop<GLU, 0>(lds, acc, st, wt, wn, fr); break;
    }

    // Epilogue.  Lane l holds, for each (j, i) and run q < 4, token
    // 32 i + (l & 31) of the wavefront's token half and weight rows
    // 32 j + 8 q + 4 (l / 32) + 0..3 of its block j.  The bf16 tile goes to
    // LDS as [256 rows][NCOLS] with 16-byte unit u of row r at unit
    // u ^ (r % OU), then leaves as whole rows, 16 bytes per thread.
    __syncthreads();   // every wavefront is done reading the k loop's stages
    const int cq = 4 * (lane >> 5);
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int trow = wt * 128 + 32 * i + (lane & 31);
      const float rs = sc_row[trow];
      uint8_t* orow = lds + trow * (NCOLS * 2);
      auto put = [&](int c, uint32_t lo, uint32_t hi) {   // c: tile column, multiple of 4
        const int u = (c >> 3) ^ (trow % OU);
        *reinterpret_cast<uint2*>(orow + u * 16 + (c & 4) * 2) = uint2{lo, hi};
      };
      if (GLU) {
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          const int c = wn * 32 + 8 * q + cq;
          float v[4];
#pragma unroll
          for (int jj = 0; jj < 4; ++jj) {
            const float hg = (float)acc[0][i][4 * q + jj] * rs * sc_col[c + jj];
            const float hu = (float)acc[1][i][4 * q + jj] * rs * sc_col[NCOLS + c + jj];
            v[jj] = ffn_silu(hg) * hu;
          }
          put(c, ffn_pack_bf16(v[0], v[1]), ffn_pack_bf16(v[2], v[3]));
        }
      } else {
#pragma unroll
        for (int j = 0; j < 2; ++j)
#pragma unroll
          for (int q = 0; q < 4; ++q) {
            const int c = wn * 64 + 32 * j + 8 * q + cq;
            float v[4];
#pragma unroll
            for (int jj = 0; jj < 4; ++jj) v[jj] = (float)acc[j][i][4 * q + jj] * rs * sc_col[c + jj];
            put(c, ffn_pack_bf16(v[0], v[1]), ffn_pack_bf16(v[2], v[3]));
          }
      }
    }
    __syncthreads();
    {
      const int u = tid % OU;
      const int col = n0 + u * 8;
#pragma unroll 4
      for (int rr = tid / OU; rr < kFfnBM; rr += kFfnThreads / OU) {
        const int row = row0 + rr;
        if (row < row_end && col < Nout) {
          const v4u v = *reinterpret_cast<const v4u*>(lds + rr * (NCOLS * 2) + ((u ^ (rr % OU)) * 16));
          *reinterpret_cast<v4u*>(out + (int64_t)row * Nout + col) = v;
        }
      }
    }
  }
}

// ---------------------------------------------------------------------------
// Host side
// ---------------------------------------------------------------------------
inline size_t round_up(size_t v, size_t a) { return (v + a - 1) / a * a; }
inline bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

mdc_status check_shape(const mdc_shape* sh) {
  if (sh == nullptr) return MDC_ERR_NULLPTR;
  if (sh->world < 1 || sh->rank < 0 || sh->rank >= sh->world) return MDC_ERR_INVALID;
  if (sh->bs < 0 || sh->hidden <= 0 || (sh->hidden % 8) != 0) return MDC_ERR_INVALID;
  if (sh->topk < 1 || sh->topk > MDC_MAX_TOPK) return MDC_ERR_INVALID;
  if (sh->num_experts <= 0 || (sh->num_experts % sh->world) != 0) return MDC_ERR_INVALID;
  if (sh->num_experts / sh->world > MDC_MAX_LOCAL_EXPERTS) return MDC_ERR_INVALID;
  if (sh->capacity < 0 || sh->capacity > INT32_MAX) return MDC_ERR_INVALID;
  if ((int64_t)sh->world * sh->bs * sh->topk > INT32_MAX) return MDC_ERR_INVALID;
  if (sh->world > 65535) return MDC_ERR_INVALID;
  if (sh->mask_per_route != 0 && sh->mask_per_route != 1) return MDC_ERR_INVALID;
  if (sh->zero_experts < 0 || sh->copy_experts < 0 || sh->reserved != 0) return MDC_ERR_INVALID;
  if ((int64_t)sh->num_experts + sh->zero_experts + sh->copy_experts > INT32_MAX) return MDC_ERR_INVALID;
  if (sh->topk > sh->num_experts + sh->zero_experts + sh->copy_experts) return MDC_ERR_INVALID;
  return MDC_OK;
}

struct DispatchPlan {
  int W, d, BS, H, K, E, L, TPG, G, nvec, rank_threads, mask_per_route;
  int64_t A;
  size_t off_p, off_cnt, bytes;
};

DispatchPlan make_plan(const mdc_shape* sh) {
  DispatchPlan p;
  p.W = sh->world;
  p.d = sh->rank;
  p.BS = sh->bs;
  p.H = sh->hidden;
  p.K = sh->topk;
  p.E = sh->num_experts;
  p.L = p.E / p.W;
  p.A = sh->capacity;
  p.mask_per_route = sh->mask_per_route;
  p.TPG = kGroupRoutes / p.K;
  p.G = (p.BS + p.TPG - 1) / p.TPG;
  p.nvec = p.H / 8;
  // wave_cnt[nw][L] + carry[L] must fit in LDS: 16 wavefronts up to L = 512, 4 beyond
  p.rank_threads = p.L <= 512 ? 1024 : 256;
  const size_t routes = (size_t)p.W * p.BS * p.K;
  const size_t counters = round_up((size_t)p.L * p.W * p.G, kScanChunk);
  p.off_p = 0;
  p.off_cnt = round_up(routes * 4, 256);
  p.bytes = p.off_cnt + round_up(counters * 4, 256);
  if (p.bytes == 0) p.bytes = 256;
  return p;
}

mdc_status launched() { return hipGetLastError() == hipSuccess ? MDC_OK : MDC_ERR_HIP; }

mdc_status layout_impl(const DispatchPlan& p, const int32_t* ids, const uint8_t* mask, char* ws, hipStream_t st) {
  int32_t* P = reinterpret_cast<int32_t*>(ws + p.off_p);
  int32_t* cnt = reinterpret_cast<int32_t*>(ws + p.off_cnt);
  if (p.G == 0) return MDC_OK;
  (void)hipGetLastError();
  const size_t lds = (size_t)(p.rank_threads / 64 + 1) * p.L * sizeof(int32_t);
  hipLaunchKernelGGL(k_route_rank, dim3(p.G, p.W), dim3(p.rank_threads), lds, st,
                     ids, mask, P, cnt, p.BS, p.K, p.E, p.L, p.d, p.W, p.TPG, p.G, p.mask_per_route);
  return launched();
}

mdc_status gather_impl(const DispatchPlan& p, const void* x, void* expand_x, int32_t* assist, int32_t* ep_recv,
                       int64_t* expert_nums, int32_t* row_idx, char* ws, hipStream_t st) {
  const int32_t* P = reinterpret_cast<const int32_t*>(ws + p.off_p);
  const int32_t* cnt = reinterpret_cast<const int32_t*>(ws + p.off_cnt);
  (void)hipGetLastError();
  const int64_t tokens = (int64_t)p.W * p.BS;
  if (tokens == 0) {
    // nothing routed: zero the counts with one wavefront of the gather kernel's writer path
    hipLaunchKernelGGL(k_zero_counts, dim3(1), dim3(64), 0, st, ep_recv, expert_nums, p.L, p.W);
    return launched();
  }
  const int ntiles = (p.nvec + 64 * kGatherVec - 1) / (64 * kGatherVec);
  const int vpl = (p.nvec + 64 * ntiles - 1) / (64 * ntiles);
  const unsigned n_items = (unsigned)(tokens * ntiles);
  const dim3 grid((n_items + MDC_GATHER_WAVES - 1) / MDC_GATHER_WAVES), block(64 * MDC_GATHER_WAVES);
#define MDC_LAUNCH_GATHER(V)                                                                                  \
  hipLaunchKernelGGL(k_dispatch_gather<V>, grid, block, 0, st, static_cast<const v4u*>(x), P, cnt,            \
                     static_cast<v4u*>(expand_x), assist, ep_recv, expert_nums, row_idx, p.BS, p.K, p.L,        \
                     p.W, p.TPG, p.G, p.A, p.nvec, ntiles, n_items)
  switch (vpl) {
    case 1: MDC_LAUNCH_GATHER(1); break;
    case 2: MDC_LAUNCH_GATHER(2); break;
    case 3: MDC_LAUNCH_GATHER(3); break;
    case 4: MDC_LAUNCH_GATHER(4); break;
    case 5: MDC_LAUNCH_GATHER(5); break;
    case 6: MDC_LAUNCH_GATHER(6); break;
    case 7: MDC_LAUNCH_GATHER(7); break;
    default: MDC_LAUNCH_GATHER(8); break;
  }
#undef MDC_LAUNCH_GATHER
  return launched();
}

mdc_status gather_q_impl(const DispatchPlan& p, const void* x, int8_t* expand_q, float* dyn_scale, int32_t* assist,
                         int32_t* ep_recv, int64_t* expert_nums, int32_t* row_idx, char* ws, hipStream_t st) {
  const int32_t* P = reinterpret_cast<const int32_t*>(ws + p.off_p);
  const int32_t* cnt = reinterpret_cast<const int32_t*>(ws + p.off_cnt);
  (void)hipGetLastError();
  const int64_t tokens = (int64_t)p.W * p.BS;
  if (tokens == 0) {
    hipLaunchKernelGGL(k_zero_counts, dim3(1), dim3(64), 0, st, ep_recv, expert_nums, p.L, p.W);
    return launched();
  }
  const int vpl = (p.nvec + 63) / 64;
#define MDC_LAUNCH_GQ(V)                                                                                          \
  hipLaunchKernelGGL(k_dispatch_gather_q<V>, dim3((unsigned)tokens), dim3(64), 0, st, static_cast<const v4u*>(x), \
                     P, cnt, expand_q, dyn_scale, assist, ep_recv, expert_nums, row_idx, p.BS, p.K, p.L, p.W,   \
                     p.TPG, p.G, p.A, p.nvec)
  if (vpl <= 4) MDC_LAUNCH_GQ(4);
  else if (vpl <= 8) MDC_LAUNCH_GQ(8);
  else if (vpl <= 12) MDC_LAUNCH_GQ(12);
  else MDC_LAUNCH_GQ(16);
#undef MDC_LAUNCH_GQ
  return launched();
}

struct FfnPlan {
  int64_t A;
  int H, N, L;
  size_t off_q1, off_s1, off_g, off_q2, off_s2, off_tiles, bytes;
};

FfnPlan make_ffn_plan(const mdc_shape* sh, int inter_n) {
  FfnPlan f;
  f.A = sh->capacity;
  f.H = sh->hidden;
  f.N = inter_n;
  f.L = sh->num_experts / sh->world;
  f.off_q1 = 0;
  f.off_s1 = round_up((size_t)f.A * f.H, 256);
  f.off_g = f.off_s1 + round_up((size_t)f.A * 4, 256);
  f.off_q2 = f.off_g + round_up((size_t)f.A * (f.N / 2) * 2, 256);
  f.off_s2 = f.off_q2 + round_up((size_t)f.A * (f.N / 2), 256);
  f.off_tiles = f.off_s2 + round_up((size_t)f.A * 4, 256);
  // m-tile table: header + at most A / kFfnBM + L tiles
  f.bytes = f.off_tiles + round_up((size_t)(2 + f.A / kFfnBM + f.L) * sizeof(int4), 256);
  if (f.bytes == 0) f.bytes = 256;
  return f;
}

mdc_status check_ffn(const mdc_shape* sh, int inter_n) {
  const mdc_status st = check_shape(sh);
  if (st != MDC_OK) return st;
  if (inter_n <= 0 || (inter_n % (2 * kFfnOutAlign)) != 0) return MDC_ERR_INVALID;
  if ((sh->hidden % kFfnOutAlign) != 0) return MDC_ERR_INVALID;
  // one expert's weight matrix (N x H or H x N/2 bytes) is addressed with 32-bit offsets
  if ((int64_t)inter_n * sh->hidden > INT32_MAX) return MDC_ERR_INVALID;
  return MDC_OK;
}

mdc_status ffn_impl(const FfnPlan& f, const void* expand_x, const int8_t* expand_q, const float* dyn_scale,
                    const int64_t* expert_token_nums, const int8_t* w1, const float* w1_scale, const int8_t* w2,
                    const float* w2_scale, void* y, char* ws, hipStream_t s) {
  int8_t* q1 = reinterpret_cast<int8_t*>(ws + f.off_q1);
  float* s1 = reinterpret_cast<float*>(ws + f.off_s1);

  uint16_t* g = reinterpret_cast<uint16_t*>(ws + f.off_g);
  int8_t* q2 = reinterpret_cast<int8_t*>(ws + f.off_q2);
  float* s2 = reinterpret_cast<float*>(ws + f.off_s2);
  int dev = 0, cus = 256;
  if (hipGetDevice(&dev) == hipSuccess) (void)hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev);
  const unsigned quant_wgs = (unsigned)(cus * 8);
  // one workgroup per CU (128 KB of LDS each)
  const unsigned g1 = (unsigned)(((cus + 7) / 8) * 8);
  const unsigned g2 = g1;
  (void)hipGetLastError();
  if (expand_q == nullptr) {
    hipLaunchKernelGGL(k_ffn_quant_rows, dim3(quant_wgs), dim3(256), 0, s, static_cast<const v4u*>(expand_x), q1,
                       s1, expert_token_nums, f.L, f.A, f.H / 8);
  } else {
    q1 = const_cast<int8_t*>(expand_q);   // rows already quantised by mdc_dispatch_quant
    s1 = const_cast<float*>(dyn_scale);
  }
  int4* tiles = reinterpret_cast<int4*>(ws + f.off_tiles);
  hipLaunchKernelGGL(k_ffn_plan, dim3(1), dim3(kPlanThreads), 0, s, expert_token_nums, f.L, f.A, tiles);
  hipLaunchKernelGGL(k_ffn_gemm<true>, dim3(g1), dim3(kFfnThreads), 0, s, q1, s1, w1, w1_scale, g, tiles, f.H, f.N,
                     f.N / 2);
  hipLaunchKernelGGL(k_ffn_quant_rows, dim3(quant_wgs), dim3(256), 0, s, reinterpret_cast<const v4u*>(g), q2, s2,
                     expert_token_nums, f.L, f.A, f.N / 2 / 8);
  hipLaunchKernelGGL(k_ffn_gemm<false>, dim3(g2), dim3(kFfnThreads), 0, s, q2, s2, w2, w2_scale,
                     static_cast<uint16_t*>(y), tiles, f.N / 2, f.H, f.H);
  return launched();
}

}  // namespace

extern "C" {

const char* mdc_status_string(mdc_status status) {
  switch (status) {
    case MDC_OK: return "MDC_OK";
    case MDC_ERR_NULLPTR: return "MDC_ERR_NULLPTR: a required pointer is NULL";
    case MDC_ERR_INVALID: return "MDC_ERR_INVALID: shape, alignment or value outside the supported range";
    case MDC_ERR_WORKSPACE: return "MDC_ERR_WORKSPACE: workspace smaller than the size query returned";
    case MDC_ERR_HIP: return "MDC_ERR_HIP: a HIP kernel launch failed";
  }
  return "unknown mdc_status";
}

int32_t mdc_abi_version(void) { return MDC_ABI_VERSION; }

mdc_status mdc_dispatch_workspace_size(const mdc_shape* shape, size_t* bytes) {
  if (bytes == nullptr) return MDC_ERR_NULLPTR;
  const mdc_status st = check_shape(shape);
  if (st != MDC_OK) return st;
  *bytes = make_plan(shape).bytes;
  return MDC_OK;
}

mdc_status mdc_dispatch_layout(const mdc_shape* shape, const int32_t* expert_ids, const uint8_t* x_active_mask,
                               void* workspace, size_t workspace_bytes, void* stream) {
  mdc_status st = check_shape(shape);
  if (st != MDC_OK) return st;
  const DispatchPlan p = make_plan(shape);
  if (workspace == nullptr) return MDC_ERR_NULLPTR;
  if (p.BS > 0 && expert_ids == nullptr) return MDC_ERR_NULLPTR;
  if (workspace_bytes < p.bytes) return MDC_ERR_WORKSPACE;
  return layout_impl(p, expert_ids, x_active_mask, static_cast<char*>(workspace), static_cast<hipStream_t>(stream));
}

mdc_status mdc_dispatch_gather(const mdc_shape* shape, const void* x, void* expand_x, int32_t* assist_info,
                               int32_t* ep_recv_counts, int64_t* expert_token_nums, int32_t* expanded_row_idx,
                               void* workspace, size_t workspace_bytes, void* stream) {
  mdc_status st = check_shape(shape);
  if (st != MDC_OK) return st;
  const DispatchPlan p = make_plan(shape);
  if (workspace == nullptr || ep_recv_counts == nullptr || expert_token_nums == nullptr) return MDC_ERR_NULLPTR;
  if (p.BS > 0 && (x == nullptr || expanded_row_idx == nullptr)) return MDC_ERR_NULLPTR;
  if (p.BS > 0 && p.A > 0 && (expand_x == nullptr || assist_info == nullptr)) return MDC_ERR_NULLPTR;
  if (!aligned16(x) || !aligned16(expand_x)) return MDC_ERR_INVALID;
  if (workspace_bytes < p.bytes) return MDC_ERR_WORKSPACE;
  return gather_impl(p, x, expand_x, assist_info, ep_recv_counts, expert_token_nums, expanded_row_idx,
                     static_cast<char*>(workspace), static_cast<hipStream_t>(stream));
}

mdc_status mdc_dispatch(const mdc_shape* shape, const void* x, const int32_t* expert_ids,
                        const uint8_t* x_active_mask, void* expand_x, int32_t* assist_info,
                        int32_t* ep_recv_counts, int64_t* expert_token_nums, int32_t* expanded_row_idx,
                        void* workspace, size_t workspace_bytes, void* stream) {
  mdc_status st = check_shape(shape);
  if (st != MDC_OK) return st;
  const DispatchPlan p = make_plan(shape);
  if (ep_recv_counts == nullptr || expert_token_nums == nullptr || workspace == nullptr) return MDC_ERR_NULLPTR;
  if (p.BS > 0 && (x == nullptr || expert_ids == nullptr || expanded_row_idx == nullptr)) return MDC_ERR_NULLPTR;
  if (p.BS > 0 && p.A > 0 && (expand_x == nullptr || assist_info == nullptr)) return MDC_ERR_NULLPTR;
  if (!aligned16(x) || !aligned16(expand_x)) return MDC_ERR_INVALID;
  if (workspace_bytes < p.bytes) return MDC_ERR_WORKSPACE;
  char* ws = static_cast<char*>(workspace);
  hipStream_t s = static_cast<hipStream_t>(stream);
  st = layout_impl(p, expert_ids, x_active_mask, ws, s);
  if (st != MDC_OK) return st;
  return gather_impl(p, x, expand_x, assist_info, ep_recv_counts, expert_token_nums, expanded_row_idx, ws, s);
}

mdc_status mdc_dispatch_quant_gather(const mdc_shape* shape, const void* x, int8_t* expand_q, float* dynamic_scales,
                                     int32_t* assist_info, int32_t* ep_recv_counts, int64_t* expert_token_nums,
                                     int32_t* expanded_row_idx, void* workspace, size_t workspace_bytes,
                                     void* stream) {
  mdc_status st = check_shape(shape);
  if (st != MDC_OK) return st;
  const DispatchPlan p = make_plan(shape);
  if (p.nvec > 64 * kQuantRowVec) return MDC_ERR_INVALID;
  if (workspace == nullptr || ep_recv_counts == nullptr || expert_token_nums == nullptr) return MDC_ERR_NULLPTR;
  if (p.BS > 0 && (x == nullptr || expanded_row_idx == nullptr)) return MDC_ERR_NULLPTR;
  if (p.BS > 0 && p.A > 0 && (expand_q == nullptr || dynamic_scales == nullptr || assist_info == nullptr))
    return MDC_ERR_NULLPTR;
  if (!aligned16(x) || !aligned16(expand_q)) return MDC_ERR_INVALID;
  if (workspace_bytes < p.bytes) return MDC_ERR_WORKSPACE;
  return gather_q_impl(p, x, expand_q, dynamic_scales, assist_info, ep_recv_counts, expert_token_nums,
                       expanded_row_idx, static_cast<char*>(workspace), static_cast<hipStream_t>(stream));
}

mdc_status mdc_dispatch_quant(const mdc_shape* shape, const void* x, const int32_t* expert_ids,
                              const uint8_t* x_active_mask, int8_t* expand_q, float* dynamic_scales,
                              int32_t* assist_info, int32_t* ep_recv_counts, int64_t* expert_token_nums,
                              int32_t* expanded_row_idx, void* workspace, size_t workspace_bytes, void* stream) {
  mdc_status st = check_shape(shape);
  if (st != MDC_OK) return st;
  const DispatchPlan p = make_plan(shape);
  if (p.nvec > 64 * kQuantRowVec) return MDC_ERR_INVALID;
  if (ep_recv_counts == nullptr || expert_token_nums == nullptr || workspace == nullptr) return MDC_ERR_NULLPTR;
  if (p.BS > 0 && (x == nullptr || expert_ids == nullptr || expanded_row_idx == nullptr)) return MDC_ERR_NULLPTR;
  if (p.BS > 0 && p.A > 0 && (expand_q == nullptr || dynamic_scales == nullptr || assist_info == nullptr))
    return MDC_ERR_NULLPTR;
  if (!aligned16(x) || !aligned16(expand_q)) return MDC_ERR_INVALID;
  if (workspace_bytes < p.bytes) return MDC_ERR_WORKSPACE;
  char* ws = static_cast<char*>(workspace);
  hipStream_t s = static_cast<hipStream_t>(stream);
  st = layout_impl(p, expert_ids, x_active_mask, ws, s);
  if (st != MDC_OK) return st;
  return gather_q_impl(p, x, expand_q, dynamic_scales, assist_info, ep_recv_counts, expert_token_nums,
                       expanded_row_idx, ws, s);
}

mdc_status mdc_combine_workspace_size(const mdc_shape* shape, size_t* bytes) {
  if (bytes == nullptr) return MDC_ERR_NULLPTR;
  const mdc_status st = check_shape(shape);
  if (st != MDC_OK) return st;
  *bytes = 0;
  return MDC_OK;
}

mdc_status mdc_combine(const mdc_shape* shape, const void* const* expand_x, const int32_t* const* assist_info,
                       const int32_t* const* ep_recv_counts, const int32_t* expanded_row_idx,
                       const int32_t* expert_ids, const float* expert_scales, const uint8_t* x_active_mask,
                       const void* shared_expert_x, const void* ori_x, void* x_out, void* workspace,
                       size_t workspace_bytes, void* stream) {
  (void)workspace;
  (void)workspace_bytes;
  mdc_status st = check_shape(shape);
  if (st != MDC_OK) return st;
  const int W = shape->world;
  if (W > MDC_MAX_COMBINE_WORLD) return MDC_ERR_INVALID;
  const int BS = shape->bs;
  if (BS == 0) return MDC_OK;
  if (expand_x == nullptr || assist_info == nullptr || ep_recv_counts == nullptr) return MDC_ERR_NULLPTR;
  if (expanded_row_idx == nullptr || expert_ids == nullptr || expert_scales == nullptr || x_out == nullptr)
    return MDC_ERR_NULLPTR;
  CombineTables tabs;
  std::memset(&tabs, 0, sizeof(tabs));
  for (int j = 0; j < W; ++j) {
    if (ep_recv_counts[j] == nullptr) return MDC_ERR_NULLPTR;
    if (shape->capacity > 0 && (expand_x[j] == nullptr || assist_info[j] == nullptr)) return MDC_ERR_NULLPTR;
    if (!aligned16(expand_x[j])) return MDC_ERR_INVALID;
    tabs.y[j] = static_cast<const v4u*>(expand_x[j]);
    tabs.assist[j] = assist_info[j];
    tabs.counts[j] = ep_recv_counts[j];
  }
  if (shape->copy_experts > 0 && ori_x == nullptr) return MDC_ERR_NULLPTR;
  if (!aligned16(shared_expert_x) || !aligned16(x_out) || !aligned16(ori_x)) return MDC_ERR_INVALID;
  const int K = shape->topk;
  const int E = shape->num_experts;
  const int L = E / W;
  const int nvec = shape->hidden / 8;
  hipStream_t s = static_cast<hipStream_t>(stream);
  const v4u* sh = static_cast<const v4u*>(shared_expert_x);
  v4u* out = static_cast<v4u*>(x_out);
  const v4u* ori = static_cast<const v4u*>(ori_x);
  const int r = shape->rank;
  const int64_t A = shape->capacity;
  (void)hipGetLastError();
  if (K <= 8) {
    const int ntiles = (nvec + 64 * kCombineVec - 1) / (64 * kCombineVec);
    const unsigned n_items = (unsigned)((int64_t)BS * ntiles);
    const dim3 grid((n_items + MDC_COMBINE_WAVES - 1) / MDC_COMBINE_WAVES), block(64 * MDC_COMBINE_WAVES);
    if (sh)
      hipLaunchKernelGGL((k_combine<8, kCombineVec, true>), grid, block, 0, s, tabs, expanded_row_idx, expert_ids,
                         expert_scales, x_active_mask, sh, ori, out, r, W, K, E, L, A, nvec, ntiles, n_items,
                         shape->mask_per_route, shape->zero_experts, shape->copy_experts);
    else
      hipLaunchKernelGGL((k_combine<8, kCombineVec, false>), grid, block, 0, s, tabs, expanded_row_idx, expert_ids,
                         expert_scales, x_active_mask, sh, ori, out, r, W, K, E, L, A, nvec, ntiles, n_items,
                         shape->mask_per_route, shape->zero_experts, shape->copy_experts);
  } else {
    const int ntiles = (nvec + 63) / 64;
    const unsigned n_items = (unsigned)((int64_t)BS * ntiles);
    const dim3 grid((n_items + MDC_COMBINE_WAVES - 1) / MDC_COMBINE_WAVES), block(64 * MDC_COMBINE_WAVES);
    if (sh)
      hipLaunchKernelGGL((k_combine<16, 1, true>), grid, block, 0, s, tabs, expanded_row_idx, expert_ids,
                         expert_scales, x_active_mask, sh, ori, out, r, W, K, E, L, A, nvec, ntiles, n_items,
                         shape->mask_per_route, shape->zero_experts, shape->copy_experts);
    else
      hipLaunchKernelGGL((k_combine<16, 1, false>), grid, block, 0, s, tabs, expanded_row_idx, expert_ids,
                         expert_scales, x_active_mask, sh, ori, out, r, W, K, E, L, A, nvec, ntiles, n_items,
                         shape->mask_per_route, shape->zero_experts, shape->copy_experts);
  }
  return launched();
}

mdc_status mdc_ffn_workspace_size(const mdc_shape* shape, int32_t inter_n, size_t* bytes) {
  if (bytes == nullptr) return MDC_ERR_NULLPTR;
  const mdc_status st = check_ffn(shape, inter_n);
  if (st != MDC_OK) return st;
  *bytes = make_ffn_plan(shape, inter_n).bytes;
  return MDC_OK;
}

mdc_status mdc_ffn(const mdc_shape* shape, int32_t inter_n, const void* expand_x, const int64_t* expert_token_nums,
                   const int8_t* w1, const float* w1_scale, const int8_t* w2, const float* w2_scale, void* y,
                   void* workspace, size_t workspace_bytes, void* stream) {
  mdc_status st = check_ffn(shape, inter_n);
  if (st != MDC_OK) return st;
  const FfnPlan f = make_ffn_plan(shape, inter_n);
  if (f.A == 0) return MDC_OK;
  if (expand_x == nullptr || expert_token_nums == nullptr || w1 == nullptr || w1_scale == nullptr ||
      w2 == nullptr || w2_scale == nullptr || y == nullptr || workspace == nullptr)
    return MDC_ERR_NULLPTR;
  if (!aligned16(expand_x) || !aligned16(w1) || !aligned16(w2) || !aligned16(y)) return MDC_ERR_INVALID;
  if (workspace_bytes < f.bytes) return MDC_ERR_WORKSPACE;
  return ffn_impl(f, expand_x, nullptr, nullptr, expert_token_nums, w1, w1_scale, w2, w2_scale, y,
                  static_cast<char*>(workspace), static_cast<hipStream_t>(stream));
}

mdc_status mdc_ffn_quant_input(const mdc_shape* shape, int32_t inter_n, const int8_t* expand_q,
                               const float* dynamic_scales, const int64_t* expert_token_nums, const int8_t* w1,
                               const float* w1_scale, const int8_t* w2, const float* w2_scale, void* y,
                               void* workspace, size_t workspace_bytes, void* stream) {
  mdc_status st = check_ffn(shape, inter_n);
  if (st != MDC_OK) return st;
  const FfnPlan f = make_ffn_plan(shape, inter_n);
  if (f.A == 0) return MDC_OK;
  if (expand_q == nullptr || dynamic_scales == nullptr || expert_token_nums == nullptr || w1 == nullptr ||
      w1_scale == nullptr || w2 == nullptr || w2_scale == nullptr || y == nullptr || workspace == nullptr)
    return MDC_ERR_NULLPTR;
  if (!aligned16(expand_q) || !aligned16(w1) || !aligned16(w2) || !aligned16(y)) return MDC_ERR_INVALID;
  if (workspace_bytes < f.bytes) return MDC_ERR_WORKSPACE;
  return ffn_impl(f, nullptr, expand_q, dynamic_scales, expert_token_nums, w1, w1_scale, w2, w2_scale, y,
                  static_cast<char*>(workspace), static_cast<hipStream_t>(stream));
}


}  // extern "C"
