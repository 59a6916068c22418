// libmdc: MoE dispatch/combine hot path for AMD Instinct MI355X (gfx950).
//
// Kernels (one GPU's share; the W expert-parallel ranks are virtual buffers):
//   k_route_rank     per chunk of one source's routes: local-route filter,
//                    wavefront-ballot multi-split rank within (source, local
//                    expert), per-chunk histogram.
//   k_route_scan     one workgroup: exclusive scan of the chunk histograms in
//                    (local expert, source, chunk) order -> chunk bases,
//                    epRecvCounts (inclusive), expertTokenNums.
//   k_dispatch_gather one workgroup per source token: reads the token's row
//                    once into registers and writes it to each of its rows on
//                    this rank (fan-out), with the (src, token, k) triplets and
//                    the route -> row inverse index.
//   k_combine        one workgroup per token of the combining rank: reads the
//                    token's K expert rows (plus the shared-expert row),
//                    accumulates in fp32 in ascending k, rounds to bf16 RNE.
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

constexpr int kRankThreads = 256;     // routes per k_route_rank workgroup (4 wavefronts)
constexpr int kScanThreads = 1024;
constexpr int kScanItems = 8;         // chunk counters per scan thread per tile
constexpr int kRowVec = 2;            // 16-byte vectors per lane per row tile
constexpr int kTileVec = 64 * kRowVec;  // 16-byte vectors per wavefront row tile
constexpr int kMaxWaves = 16;

__device__ __forceinline__ uint64_t lanes_below(int lane) { return (1ull << lane) - 1ull; }

// ---------------------------------------------------------------------------
// a1 + a3 (local part): filter, per-chunk histogram, rank within chunk.
//
// A chunk is CT = floor(256 / K) consecutive tokens of one source rank, so a
// chunk never splits a token's K routes and holds at most 256 routes, one per
// thread.  Thread i handles flattened route f = t*K + k of the chunk.  Its key
// is the local expert le = e - d*L when the route is sent to rank d, or L
// otherwise.  Ranks within a wavefront come from a ballot per key bit (a
// multi-split): the lanes holding the same key form a mask, and the rank is
// the number of such lanes below.  Wavefront counts are prefixed in LDS over
// the four wavefronts, which keeps the (t, k) order: rank = number of earlier
// routes of this source and chunk with the same expert ([TL] send loop,
// rank-within-expert counts earlier equal ids).
//
// P[f] = le | (rank_in_chunk << 16) for a route sent to d, else -1.
// ---------------------------------------------------------------------------
__global__ __launch_bounds__(kRankThreads) void k_route_rank(
    const int32_t* __restrict__ ids, const uint8_t* __restrict__ mask,
    int32_t* __restrict__ P, int32_t* __restrict__ chunk_cnt,
    int BS, int K, int E, int L, int d, int CT, int nC) {
  extern __shared__ int32_t wave_cnt[];  // [4][L]
  const int s = blockIdx.y;
  const int c = blockIdx.x;
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wv = tid >> 6;
  const int t0 = c * CT;
  const int nt = min(CT, BS - t0);
  const int nroutes = nt * K;
  const int64_t f = ((int64_t)s * BS + t0) * K + tid;

  int key = L;
  if (tid < nroutes) {
    const int t = t0 + tid / K;
    const int e = ids[f];
    const bool active = (mask == nullptr) || (mask[(int64_t)s * BS + t] != 0);
    const int q = e - d * L;
    if (active && e >= 0 && e < E && q >= 0 && q < L) key = q;
  }
  for (int i = tid; i < 4 * L; i += kRankThreads) wave_cnt[i] = 0;

  uint64_t same = __ballot(1);
  const int nbits = 32 - __clz(L);
  for (int b = 0; b < nbits; ++b) {
    const int bit = (key >> b) & 1;
    const uint64_t bal = __ballot(bit);
    same &= bit ? bal : ~bal;
  }
  const int rank_in_wave = __popcll(same & lanes_below(lane));
  __syncthreads();
  if (key < L && rank_in_wave == 0) wave_cnt[wv * L + key] = __popcll(same);
  __syncthreads();
  for (int le = tid; le < L; le += kRankThreads) {
    int run = 0;
#pragma unroll
    for (int w = 0; w < 4; ++w) {
      const int v = wave_cnt[w * L + le];
      wave_cnt[w * L + le] = run;
      run += v;
    }
    chunk_cnt[((int64_t)s * nC + c) * L + le] = run;
  }
  __syncthreads();
  if (tid < nroutes) {
    P[f] = (key < L) ? (key | ((wave_cnt[wv * L + key] + rank_in_wave) << 16)) : -1;
  }
}

__device__ __forceinline__ int wave_inclusive_scan(int v, int lane) {
#pragma unroll
  for (int o = 1; o < 64; o <<= 1) {
    const int u = __shfl_up(v, o, 64);
    if (lane >= o) v += u;
  }
  return v;
}

// ---------------------------------------------------------------------------
// a2: scan.  Items are the chunk counters in (le, s, c) order, so the
// exclusive prefix of item (le, s, c) is the first row of that chunk's routes
// to le.  The inclusive prefix at the last chunk of (le, s) is
// epRecvCounts[le*W + s] ([TL] GetCumSum and local data copy: receive count
// = begin + count); expertTokenNums[le] is the difference of consecutive
// inclusive prefixes at the end of each le block ([TL] UpdateTokenNumsOut).
// ---------------------------------------------------------------------------
__global__ __launch_bounds__(kScanThreads) void k_route_scan(
    const int32_t* __restrict__ chunk_cnt, int32_t* __restrict__ chunk_base,
    int32_t* __restrict__ ep_recv, int64_t* __restrict__ expert_nums,
    int W, int L, int nC) {
  extern __shared__ int32_t le_end[];  // [L]
  __shared__ int32_t wave_tot[kScanThreads / 64];
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wv = tid >> 6;
  const int64_t per_le = (int64_t)W * nC;
  const int64_t N = per_le * L;

  for (int i = tid; i < L; i += kScanThreads) le_end[i] = 0;
  if (nC == 0) {
    for (int64_t i = tid; i < (int64_t)L * W; i += kScanThreads) ep_recv[i] = 0;
  }
  __syncthreads();

  int carry = 0;
  for (int64_t tile = 0; tile < N; tile += (int64_t)kScanThreads * kScanItems) {
    int vals[kScanItems];
    int sum = 0;
#pragma unroll
    for (int j = 0; j < kScanItems; ++j) {
      const int64_t q = tile + (int64_t)tid * kScanItems + j;
      int v = 0;
      if (q < N) {
        const int le = (int)(q / per_le);
        const int64_t rem = q - (int64_t)le * per_le;
        const int s = (int)(rem / nC);
        const int c = (int)(rem - (int64_t)s * nC);
        v = chunk_cnt[((int64_t)s * nC + c) * L + le];
      }
      vals[j] = v;
      sum += v;
    }
    const int incl = wave_inclusive_scan(sum, lane);
    if (lane == 63) wave_tot[wv] = incl;
    __syncthreads();
    int wave_off = 0;
    int tile_tot = 0;
#pragma unroll
    for (int w = 0; w < kScanThreads / 64; ++w) {
      const int x = wave_tot[w];
      wave_off += (w < wv) ? x : 0;
      tile_tot += x;
    }
    int run = carry + wave_off + incl - sum;
#pragma unroll
    for (int j = 0; j < kScanItems; ++j) {
      const int64_t q = tile + (int64_t)tid * kScanItems + j;
      if (q < N) {
        const int le = (int)(q / per_le);
        const int64_t rem = q - (int64_t)le * per_le;
        const int s = (int)(rem / nC);
        const int c = (int)(rem - (int64_t)s * nC);
        chunk_base[((int64_t)s * nC + c) * L + le] = run;
        if (c == nC - 1) {
          ep_recv[(int64_t)le * W + s] = run + vals[j];
          if (s == W - 1) le_end[le] = run + vals[j];
        }
      }
      run += vals[j];
    }
    carry += tile_tot;
    __syncthreads();
  }
  for (int le = tid; le < L; le += kScanThreads) {
    expert_nums[le] = (int64_t)le_end[le] - (le > 0 ? le_end[le - 1] : 0);
  }
}

// ---------------------------------------------------------------------------
// a3 (global rows) + a4 + a5: one workgroup per source token g = s*BS + t.
// Lanes 0..K-1 turn the token's ranks into rows (chunk base + rank in chunk),
// rows at or beyond the capacity are dropped.  Wavefront 0 writes the
// triplets and the inverse index.  Each wavefront then copies its column
// tiles of x[s][t]: one read, one non-temporal write per destination row
// ([TL] send loop row put and local data copy; [PTO] Dispatch Stage pull).
// ---------------------------------------------------------------------------
__global__ __launch_bounds__(1024) void k_dispatch_gather(
    const v4u* __restrict__ x, const int32_t* __restrict__ P,
    const int32_t* __restrict__ chunk_base, v4u* __restrict__ expand_x,
    int32_t* __restrict__ assist, int32_t* __restrict__ row_idx,
    int BS, int K, int L, int CT, int nC, int64_t A, int nvec) {
  const int64_t g = blockIdx.x;
  const int s = (int)(g / BS);
  const int t = (int)(g - (int64_t)s * BS);
  const int lane = threadIdx.x & 63;
  const int wv = threadIdx.x >> 6;
  const int nw = blockDim.x >> 6;

  // A route is ours when its packed entry holds a local expert < L; the row
  // is kept only inside [0, A), so a stale workspace can never address
  // memory outside the outputs.
  bool mine = false;
  int row = -1;
  if (lane < K) {
    const int p = P[g * K + lane];
    if (p >= 0 && (p & 0xFFFF) < L) {
      mine = true;
      const int le = p & 0xFFFF;
      const int rk = p >> 16;
      const int64_t r = (int64_t)chunk_base[((int64_t)s * nC + t / CT) * L + le] + rk;
      row = (r >= 0 && r < A) ? (int)r : -1;
    }
  }
  if (wv == 0 && mine) {
    row_idx[g * K + lane] = row;
    if (row >= 0) {
      int32_t* a = assist + (int64_t)row * 3;
      a[0] = s;
      a[1] = t;
      a[2] = lane;
    }
  }
  const uint64_t has = __ballot(row >= 0);
  if (has == 0) return;

  const v4u* src = x + g * nvec;
  for (int tile = wv; tile * kTileVec < nvec; tile += nw) {
    const int base = tile * kTileVec + lane;
    v4u v[kRowVec];
#pragma unroll
    for (int u = 0; u < kRowVec; ++u) {
      const int idx = base + u * 64;
      if (idx < nvec) v[u] = src[idx];
    }
    uint64_t rem = has;
    while (rem) {
      const int k = __ffsll((unsigned long long)rem) - 1;
      rem &= rem - 1;
      const int rk = __builtin_amdgcn_readlane(row, k);
      v4u* dst = expand_x + (int64_t)rk * nvec;
#pragma unroll
      for (int u = 0; u < kRowVec; ++u) {
        const int idx = base + u * 64;
        if (idx < nvec) __builtin_nontemporal_store(v[u], dst + idx);
      }
    }
  }
}

// ---------------------------------------------------------------------------
// a6: combine.  One workgroup per token t of rank r.
// ---------------------------------------------------------------------------
struct CombineTables {
  const v4u* y[MDC_MAX_COMBINE_WORLD];
  const int32_t* assist[MDC_MAX_COMBINE_WORLD];
  const int32_t* counts[MDC_MAX_COMBINE_WORLD];
};

__device__ __forceinline__ float bf16_lo(unsigned w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf16_hi(unsigned w) { return __uint_as_float(w & 0xFFFF0000u); }

// fp32 -> bf16 round to nearest, ties to even (the CAST_RINT of [TL] combine):
// add 0x7FFF plus the lowest kept bit, keep the top 16 bits; NaN -> quiet NaN.
__device__ __forceinline__ unsigned bf16_rne(float f) {
  const unsigned u = __float_as_uint(f);
  if (f != f) return ((u >> 16) & 0x8000u) | 0x7FC0u;
  return (u + 0x7FFFu + ((u >> 16) & 1u)) >> 16;
}

__device__ __forceinline__ uint64_t readlane64(uint64_t v, int k) {
  const unsigned lo = (unsigned)__builtin_amdgcn_readlane((int)(unsigned)v, k);
  const unsigned hi = (unsigned)__builtin_amdgcn_readlane((int)(unsigned)(v >> 32), k);
  return ((uint64_t)hi << 32) | lo;
}

template <int KMAX, bool SHARED>
__global__ __launch_bounds__(1024) void k_combine(
    CombineTables tabs, const int32_t* __restrict__ row_idx, const int32_t* __restrict__ ids,
    const float* __restrict__ scales, const uint8_t* __restrict__ mask,
    const v4u* __restrict__ shared, v4u* __restrict__ out,
    int r, int W, int K, int E, int L, int64_t A, int nvec) {
  const int t = blockIdx.x;
  const int lane = threadIdx.x & 63;
  const int wv = threadIdx.x >> 6;
  const int nw = blockDim.x >> 6;

  // Lane k < K resolves route (r, t, k): destination j = e / L, row from the
  // inverse index, checked against that destination's count and triplet.
  bool ok = false;
  uint64_t yrow = 0;
  float sc = 0.f;
  if (lane < K && (mask == nullptr || mask[t] != 0)) {
    const int e = ids[(int64_t)t * K + lane];
    if (e >= 0 && e < E) {
      const int j = e / L;
      const int row = row_idx[(int64_t)t * K + lane];
      const int64_t total = tabs.counts[j][(int64_t)L * W - 1];
      const int64_t lim = total < A ? total : A;
      if (row >= 0 && row < lim) {
        const int32_t* a = tabs.assist[j] + (int64_t)row * 3;
        if (a[0] == r && a[1] == t && a[2] == lane) {
          ok = true;
          yrow = (uint64_t)(tabs.y[j] + (int64_t)row * nvec);
          sc = scales[(int64_t)t * K + lane];
        }
      }
    }
  }
  const uint64_t has = __ballot(ok);
  const int np = __popcll(has);

  // Present routes in ascending k, as wavefront-uniform pointers and scales.
  const v4u* yp[KMAX];
  float sk[KMAX];
  uint64_t rem = has;
#pragma unroll
  for (int i = 0; i < KMAX; ++i) {
    const int k = rem ? (__ffsll((unsigned long long)rem) - 1) : 0;
    yp[i] = (const v4u*)readlane64(yrow, k);
    sk[i] = __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, sc), k));
    rem &= rem - 1;
  }

  const v4u* shrow = SHARED ? shared + (int64_t)t * nvec : nullptr;
  v4u* orow = out + (int64_t)t * nvec;
  for (int tile = wv; tile * kTileVec < nvec; tile += nw) {
    const int base = tile * kTileVec + lane;
    v4u yv[KMAX][kRowVec];
    v4u shv[kRowVec];
#pragma unroll
    for (int i = 0; i < KMAX; ++i) {
      if (i < np) {
#pragma unroll
        for (int u = 0; u < kRowVec; ++u) {
          const int idx = base + u * 64;
          if (idx < nvec) yv[i][u] = yp[i][idx];
        }
      }
    }
    if (SHARED && np > 0) {
#pragma unroll
      for (int u = 0; u < kRowVec; ++u) {
        const int idx = base + u * 64;
        if (idx < nvec) shv[u] = shrow[idx];
      }
    }
#pragma unroll
    for (int u = 0; u < kRowVec; ++u) {
      const int idx = base + u * 64;
      if (idx >= nvec) continue;
      float acc[8];
#pragma unroll
      for (int e = 0; e < 8; ++e) acc[e] = 0.f;
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
      __builtin_nontemporal_store(o, orow + idx);
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
  return MDC_OK;
}

struct DispatchPlan {
  int W, d, BS, H, K, E, L, CT, nC, nvec;
  int64_t A;
  size_t off_p, off_cnt, off_base, bytes;
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
  p.CT = kRankThreads / p.K;
  p.nC = (p.BS + p.CT - 1) / p.CT;
  p.nvec = p.H / 8;
  const size_t routes = (size_t)p.W * p.BS * p.K;
  const size_t chunks = (size_t)p.W * p.nC * p.L;
  p.off_p = 0;
  p.off_cnt = round_up(routes * 4, 256);
  p.off_base = p.off_cnt + round_up(chunks * 4, 256);
  p.bytes = p.off_base + round_up(chunks * 4, 256);
  if (p.bytes == 0) p.bytes = 256;
  return p;
}

int row_waves(int nvec) {
  int tiles = (nvec + kTileVec - 1) / kTileVec;
  return tiles < kMaxWaves ? tiles : kMaxWaves;
}

mdc_status launched() { return hipGetLastError() == hipSuccess ? MDC_OK : MDC_ERR_HIP; }

mdc_status layout_impl(const DispatchPlan& p, const int32_t* ids, const uint8_t* mask,
                       int32_t* ep_recv, int64_t* expert_nums, char* ws, hipStream_t st) {
  int32_t* P = reinterpret_cast<int32_t*>(ws + p.off_p);
  int32_t* cnt = reinterpret_cast<int32_t*>(ws + p.off_cnt);
  int32_t* base = reinterpret_cast<int32_t*>(ws + p.off_base);
  (void)hipGetLastError();
  if (p.nC > 0) {
    hipLaunchKernelGGL(k_route_rank, dim3(p.nC, p.W), dim3(kRankThreads), 4 * p.L * sizeof(int32_t), st,
                       ids, mask, P, cnt, p.BS, p.K, p.E, p.L, p.d, p.CT, p.nC);
  }
  hipLaunchKernelGGL(k_route_scan, dim3(1), dim3(kScanThreads), p.L * sizeof(int32_t), st,
                     cnt, base, ep_recv, expert_nums, p.W, p.L, p.nC);
  return launched();
}

mdc_status gather_impl(const DispatchPlan& p, const void* x, void* expand_x, int32_t* assist,
                       int32_t* row_idx, char* ws, hipStream_t st) {
  const int32_t* P = reinterpret_cast<const int32_t*>(ws + p.off_p);
  const int32_t* base = reinterpret_cast<const int32_t*>(ws + p.off_base);
  const int64_t tokens = (int64_t)p.W * p.BS;
  if (tokens == 0) return MDC_OK;
  (void)hipGetLastError();
  hipLaunchKernelGGL(k_dispatch_gather, dim3((unsigned)tokens), dim3(64 * row_waves(p.nvec)), 0, st,
                     static_cast<const v4u*>(x), P, base, static_cast<v4u*>(expand_x), assist, row_idx,
                     p.BS, p.K, p.L, p.CT, p.nC, p.A, p.nvec);
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

mdc_status mdc_dispatch_layout(const mdc_shape* shape, const int32_t* expert_ids,
                               const uint8_t* x_active_mask, int32_t* ep_recv_counts,
                               int64_t* expert_token_nums, void* workspace, size_t workspace_bytes,
                               void* stream) {
  mdc_status st = check_shape(shape);
  if (st != MDC_OK) return st;
  const DispatchPlan p = make_plan(shape);
  if (ep_recv_counts == nullptr || expert_token_nums == nullptr || workspace == nullptr) return MDC_ERR_NULLPTR;
  if (p.BS > 0 && expert_ids == nullptr) return MDC_ERR_NULLPTR;
  if (workspace_bytes < p.bytes) return MDC_ERR_WORKSPACE;
  return layout_impl(p, expert_ids, x_active_mask, ep_recv_counts, expert_token_nums,
                     static_cast<char*>(workspace), static_cast<hipStream_t>(stream));
}

mdc_status mdc_dispatch_gather(const mdc_shape* shape, const void* x, void* expand_x, int32_t* assist_info,
                               int32_t* expanded_row_idx, void* workspace, size_t workspace_bytes,
                               void* stream) {
  mdc_status st = check_shape(shape);
  if (st != MDC_OK) return st;
  const DispatchPlan p = make_plan(shape);
  if (workspace == nullptr) return MDC_ERR_NULLPTR;
  if (p.BS > 0 && (x == nullptr || expanded_row_idx == nullptr)) return MDC_ERR_NULLPTR;
  if (p.BS > 0 && p.A > 0 && (expand_x == nullptr || assist_info == nullptr)) return MDC_ERR_NULLPTR;
  if (!aligned16(x) || !aligned16(expand_x)) return MDC_ERR_INVALID;
  if (workspace_bytes < p.bytes) return MDC_ERR_WORKSPACE;
  return gather_impl(p, x, expand_x, assist_info, expanded_row_idx, static_cast<char*>(workspace),
                     static_cast<hipStream_t>(stream));
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
  st = layout_impl(p, expert_ids, x_active_mask, ep_recv_counts, expert_token_nums, ws, s);
  if (st != MDC_OK) return st;
  return gather_impl(p, x, expand_x, assist_info, expanded_row_idx, ws, s);
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
                       const void* shared_expert_x, void* x_out, void* workspace, size_t workspace_bytes,
                       void* stream) {
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
  if (!aligned16(shared_expert_x) || !aligned16(x_out)) return MDC_ERR_INVALID;
  const int K = shape->topk;
  const int E = shape->num_experts;
  const int L = E / W;
  const int nvec = shape->hidden / 8;
  const dim3 grid(BS), block(64 * row_waves(nvec));
  hipStream_t s = static_cast<hipStream_t>(stream);
  const v4u* sh = static_cast<const v4u*>(shared_expert_x);
  v4u* out = static_cast<v4u*>(x_out);
  (void)hipGetLastError();
  if (K <= 8) {
    if (sh)
      hipLaunchKernelGGL((k_combine<8, true>), grid, block, 0, s, tabs, expanded_row_idx, expert_ids,
                         expert_scales, x_active_mask, sh, out, shape->rank, W, K, E, L, shape->capacity, nvec);
    else
      hipLaunchKernelGGL((k_combine<8, false>), grid, block, 0, s, tabs, expanded_row_idx, expert_ids,
                         expert_scales, x_active_mask, sh, out, shape->rank, W, K, E, L, shape->capacity, nvec);
  } else {
    if (sh)
      hipLaunchKernelGGL((k_combine<16, true>), grid, block, 0, s, tabs, expanded_row_idx, expert_ids,
                         expert_scales, x_active_mask, sh, out, shape->rank, W, K, E, L, shape->capacity, nvec);
    else
      hipLaunchKernelGGL((k_combine<16, false>), grid, block, 0, s, tabs, expanded_row_idx, expert_ids,
                         expert_scales, x_active_mask, sh, out, shape->rank, W, K, E, L, shape->capacity, nvec);
  }
  return launched();
}

}  // extern "C"
