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
//                     expertTokenNums.  The tile size follows the token's
//                     number of rows here (half rows for 1-2, 2 KB for more).
//                     (mdc_dispatch_gather)
//   k_dispatch_gather_q  as k_dispatch_gather with one wavefront per whole
//                     row, writing each row as int8 codes plus a per-row
//                     fp32 scale.  (mdc_dispatch_quant_gather)
//   k_dispatch_small  decode-size batches: all of the above in one launch,
//                     every workgroup counting, over the whole route list,
//                     the routes placed before each of its token's routes
//                     (ballots, no histogram).  (mdc_dispatch and
//                     mdc_dispatch_quant when the route list is small)
//   k_combine         one wavefront per (token, column tile) of the combining
//                     rank: reads the token's present expert rows (and the
//                     shared-expert row), accumulates in fp32 in ascending k,
//                     rounds to bf16 nearest-even.  (mdc_combine)
//
// Sources: "dispatch_combine_shmem.py" (TileLang-Ascend example),
// moe_dispatch_kernel / moe_combine_kernel; "aclnnMoeDistributeCombineV4",
// Function formula, Function Prototype and parameter notes (2D mask,
// zero/copy experts, quantised communication); "PTO MegaMoE Dispatch +
// Combine Fusion Example", FrontReorder / Dispatch / Combine / Unpermute
// stages.
//
// Built with -ffp-contract=off: the combine's products and sums are rounded
// to fp32 one by one, in the order the combine formula lists them.

#include <mutex>

#include "mdc_route.h"

// Workspace of mdc_dispatch_noalloc, for callers that cannot allocate: one
// copy per device, zero at load, held until the process ends.  Host code
// never passes this name to a kernel (on the host it is only a stand-in for
// the symbol); it uses the device address from noalloc_scratch() instead.
static __device__ __align__(256) unsigned char scratch[MDC_NOALLOC_SCRATCH_BYTES];

namespace {

// Build-time tile shapes (16-byte vectors per lane per row tile).
#ifndef MDC_GATHER_VEC
#define MDC_GATHER_VEC 8
#endif
#ifndef MDC_GATHER_SMALL_VEC
#define MDC_GATHER_SMALL_VEC 2
#endif
#ifndef MDC_GATHER_FANOUT_SPLIT
#define MDC_GATHER_FANOUT_SPLIT 2
#endif
#ifndef MDC_COMBINE_VEC
#define MDC_COMBINE_VEC 1
#endif
// Cache policy per kernel (1 = non-temporal).  Measured on MI355X over whole
// dispatch+combine steps: non-temporal row loads and stores in both kernels
// give the shortest step (the two kernels share the Infinity Cache, so each
// one's policy also moves the other's time).  The quantised gather's int8
// rows are the exception: they are stored with the default policy, which
// is faster for its 8-byte stores and leaves the rows cached for the GEMM
// that reads them next (MDC_GATHER_Q_NT_STORES).
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
#ifndef MDC_GATHER_Q_NT_STORES
#define MDC_GATHER_Q_NT_STORES 0
#endif
#ifndef MDC_COMBINE_NT_LOADS
#define MDC_COMBINE_NT_LOADS 1
#endif
#ifndef MDC_COMBINE_NT_STORES
#define MDC_COMBINE_NT_STORES 1
#endif
constexpr int kGatherVec = MDC_GATHER_VEC;
constexpr int kGatherSmallVec = MDC_GATHER_SMALL_VEC;      // tile of the tokens with many rows here
static_assert(kGatherSmallVec >= 1 && kGatherSmallVec < 5, "small tiles must be smaller than the tiles they replace");
constexpr int kGatherFanoutSplit = MDC_GATHER_FANOUT_SPLIT;  // more rows than this: small tiles
static_assert(kGatherVec >= 1 && kGatherVec <= 8, "gather tiles hold 1..8 vectors per lane");
constexpr int kCombineVec = MDC_COMBINE_VEC;

// ---------------------------------------------------------------------------
// a1 + a3 (ranks): route filter, histogram and stable rank within a group.
//
// A group is TPG = floor(kGroupRoutes / K) consecutive tokens of one source rank; one
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
// drop[s*G + g] = active routes of the group whose id lies outside [0, n_ids),
// n_ids = E + Z + C (sent nowhere; reported in the status block).
// ---------------------------------------------------------------------------
__global__ __launch_bounds__(1024) void k_route_rank(
    const int32_t* __restrict__ ids, const uint8_t* __restrict__ mask,
    int32_t* __restrict__ P, int32_t* __restrict__ cnt, int32_t* __restrict__ drop,
    int BS, int K, int E, int L, int d, int W, int TPG, int G, int mask_per_route, int n_ids) {
  extern __shared__ int32_t sm[];  // carry[L], wave_cnt[nw][L]
  __shared__ int32_t drop_s;
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
  int dropped = 0;
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
      dropped += (active && (e < 0 || e >= n_ids)) ? 1 : 0;
    }
    keys[i] = key;
  }
  for (int i = tid; i < L; i += blockDim.x) carry[i] = 0;
  if (tid == 0) drop_s = 0;
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
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) dropped += __shfl_xor(dropped, o, 64);
  if (lane == 0 && dropped != 0) atomicAdd(&drop_s, dropped);
  __syncthreads();
  if (tid == 0) drop[s * G + g] = drop_s;
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
                           bool writer, int32_t* __restrict__ ep_recv, int lane, int32_t* __restrict__ pref,
                           int& total) {
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
  total = carry;
  return found;
}

// The writer wavefront's part of the counts: expertTokenNums[le] = sum of the
// group counters of le ([TL] UpdateTokenNumsOut), and the status block:
// dropped ids summed over the rank groups, rows past the capacity.
__device__ void write_totals(const int32_t* __restrict__ cnt, const int32_t* __restrict__ drop,
                             int64_t* __restrict__ expert_nums, mdc_device_status* __restrict__ status, int L,
                             int W, int G, int total, int64_t A, int lane) {
  for (int e = lane; e < L; e += 64) {
    int64_t sum = 0;
    for (int i = 0; i < W * G; ++i) sum += cnt[counter_slot(e * W * G + i)];
    expert_nums[e] = sum;
  }
  int dropped = 0;
  for (int i = lane; i < W * G; i += 64) dropped += drop[i];
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) dropped += __shfl_xor(dropped, o, 64);
  if (lane == 0) {
    const int64_t over = (int64_t)total - A;
    status->dropped_ids = dropped;
    status->overflow_rows = over > 0 ? (int32_t)over : 0;
    status->wait_timeouts = 0;
    status->reserved = 0;
  }
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
// One column tile (64 * V vectors from `tile * 64 * V`) of token g's row:
// loads it, finds the token's rows (in-wavefront scan of the group
// counters) and writes the tile to each of them; tile 0 also writes the
// triplets and inverse-index entries, and the writer wavefront the counts.

template <int V>
__device__ __forceinline__ void gather_tile(
    const v4u* __restrict__ x, const GatherMeta& m, v4u* __restrict__ expand_x,
    int64_t g, int s, int t, int tile, int lane, int p, bool mine, uint64_t has,
    bool writer, int K, int L, int W, int TPG, int G, int64_t A, int nvec, int32_t* pref) {
  const int32_t* __restrict__ cnt = m.cnt;
  const int n_cnt = L * W * G;
  int cnt0[kScanIPL];
  load_counters(cnt, n_cnt, 0, lane, cnt0);

  // Column tile of the source row: issued before the scan so the loads overlap it.
  const int base = tile * 64 * V + lane;
  const bool full = (tile + 1) * 64 * V <= nvec;
  const uint64_t src = (uint64_t)(x + g * nvec);
  v4u v[V];
  if (has != 0) {
    if (full) {
#pragma unroll
      for (int u = 0; u < V; ++u) v[u] = load_v4<MDC_GATHER_NT_LOADS != 0>(src + (uint64_t)(base + u * 64) * 16);
    } else {
#pragma unroll
      for (int u = 0; u < V; ++u) {
        const int idx = base + u * 64;
        v[u] = idx < nvec ? load_v4<MDC_GATHER_NT_LOADS != 0>(src + (uint64_t)idx * 16) : v4u{0u, 0u, 0u, 0u};
      }
    }
  }

  const int le = p & 0xFFFF;
  const int q = mine ? ((le * W + s) * G + t / TPG) : -1;
  int total;
  const int first = scan_lookup(cnt, n_cnt, cnt0, q, G, writer, m.ep_recv, lane, pref, total);
  if (writer) write_totals(cnt, m.drop, m.expert_nums, m.status, L, W, G, total, A, lane);
  if (has == 0) return;

  int row = -1;
  if (mine) {
    const int64_t r = (int64_t)first + (p >> 16);
    row = (r >= 0 && r < A) ? (int)r : -1;
  }
  if (tile == 0 && mine) place_route(m, g, K, s, t, lane, row);
  uint64_t rem = __ballot(row >= 0);
  while (rem) {
    const int k = __ffsll((unsigned long long)rem) - 1;
    rem &= rem - 1;
    const int rk = __builtin_amdgcn_readlane(row, k);
    v4u* dst = expand_x + (int64_t)rk * nvec;
    if (full) {
#pragma unroll
      for (int u = 0; u < V; ++u) store_v4<MDC_GATHER_NT_STORES != 0>(dst + base + u * 64, v[u]);
    } else {
#pragma unroll
      for (int u = 0; u < V; ++u) {
        const int idx = base + u * 64;
        if (idx < nvec) store_v4<MDC_GATHER_NT_STORES != 0>(dst + idx, v[u]);
      }
    }
  }
}

// The launch has ntiles items per token: tiles of 64 * VS vectors.  A token
// with more than kGatherFanoutSplit rows on this rank uses them all; one with
// fewer uses the first ceil(nvec / (64 * VPL)) items for tiles of 64 * VPL
// vectors and the others return.  (With VS == VPL every token uses tiles of
// 64 * VPL vectors.)  Measured at the share shapes: with 5 rows per source
// token (Zipf routes) 2-vector tiles are 13% faster than 7-vector ones, with
// 1.5 rows per token 11% slower.
template <int VPL, int VS>
__global__ __launch_bounds__(64 * MDC_GATHER_WAVES) void k_dispatch_gather(
    const v4u* __restrict__ x, GatherMeta m, v4u* __restrict__ expand_x,
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
  const int p = (lane < K) ? m.P[g * K + lane] : -1;
  const bool mine = (p >= 0) && ((p & 0xFFFF) < L);
  const uint64_t has = __ballot(mine);
  if (has == 0 && !writer) return;
  __shared__ int32_t pref_all[MDC_GATHER_WAVES][kScanChunk];
  int32_t* pref = pref_all[threadIdx.x >> 6];
  if (VS < VPL && __popcll(has) > kGatherFanoutSplit) {
    gather_tile<VS>(x, m, expand_x, g, s, t, tile, lane, p, mine, has, writer, K, L, W, TPG, G, A, nvec, pref);
    return;
  }
  if (VS < VPL && tile * 64 * VPL >= nvec) return;   // (tile 0, the writer's, always has vectors)
  gather_tile<VPL>(x, m, expand_x, g, s, t, tile, lane, p, mine, has, writer, K, L, W, TPG, G, A, nvec, pref);
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

template <int VPL>
__global__ __launch_bounds__(64) void k_dispatch_gather_q(
    const v4u* __restrict__ x, GatherMeta m, int8_t* __restrict__ expand_q, float* __restrict__ dyn_scale,
    int BS, int K, int L, int W, int TPG, int G, int64_t A, int nvec) {
  const int32_t* __restrict__ cnt = m.cnt;
  const unsigned gu = blockIdx.x;
  const int s = (int)(gu / (unsigned)BS);
  const int t = (int)(gu - (unsigned)s * (unsigned)BS);
  const int64_t g = gu;
  const int lane = threadIdx.x & 63;
  const bool writer = (g == 0);
  const int n_cnt = L * W * G;
  int cnt0[kScanIPL];
  load_counters(cnt, n_cnt, 0, lane, cnt0);
  const int p = (lane < K) ? m.P[g * K + lane] : -1;
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
  int total;
  const int first = scan_lookup(cnt, n_cnt, cnt0, q, G, writer, m.ep_recv, lane, pref_all, total);
  if (writer) write_totals(cnt, m.drop, m.expert_nums, m.status, L, W, G, total, A, lane);
  if (has == 0) return;

  uint64_t qv[VPL];
  const float scale = quant_row<VPL>(v, qv);

  int row = -1;
  if (mine) {
    const int64_t r = (int64_t)first + (p >> 16);
    row = (r >= 0 && r < A) ? (int)r : -1;
  }
  if (mine) {
    place_route(m, g, K, s, t, lane, row);
    if (row >= 0) dyn_scale[row] = scale;
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
        if (MDC_GATHER_Q_NT_STORES) __builtin_nontemporal_store(qv[u], dst + idx);
        else dst[idx] = qv[u];
      }
    }
  }
}

// ---------------------------------------------------------------------------
// Small batches: a1 - a5 in one launch.  When the whole route list is small
// (decode-size batches), every workgroup reads all route ids and counts what
// it needs instead of building the histogram and its scan.  In the stable
// expert-major (source, token, k) order, the row of route f with local
// expert e is the number of routes sent here with a smaller local expert
// plus the number with expert e that come before f ([TL] GetCumSum and the
// send loop's ranks, taken together); epRecvCounts[e][s] is the inclusive
// count of routes with a smaller expert, or expert e from sources <= s, and
// expertTokenNums[e] the number with expert e.  Each wavefront counts with
// one ballot per route id it holds and the workgroup sums the wavefronts'
// counts: no atomics, no scan, two barriers.  Workgroup b places its own
// token's routes and copies (QUANT: quantises) the token's row, and also
// writes epRecvCounts entry r G + b and expertTokenNums entry
// r G + G - 1 - b for rounds r = 0, 1, ... while they exist (G workgroups,
// one per source token), so that no workgroup counts much more than another;
// the last epRecvCounts entry is the number of routes sent here, from which
// its workgroup writes the overflow count, and workgroup 0 counts the
// dropped ids.  One 512-thread workgroup per source token.  This replaces
// the rank kernel and the gather kernel; the outputs are identical.
// ---------------------------------------------------------------------------
constexpr int kSmallRoutes = 8192;                  // route ids every workgroup reads
constexpr int kSmallMaxRounds = 16;                 // epRecvCounts entries per workgroup
constexpr int64_t kSmallRereads = int64_t(1) << 20; // tokens x routes: ids every workgroup rereads
constexpr int kSmallThreads = 512;
constexpr int kSmallRowVec = 2;                     // row vectors per thread kept for the quantiser
constexpr int kSmallKeyBatch = 4;                   // route ids per thread per batch of kSmallThreads * 4
// counted values per round: the token's routes, the round's epRecvCounts
// entry and expert count, and (workgroup 0) the dropped ids
constexpr int kSmallSlotCnt = MDC_MAX_TOPK;
constexpr int kSmallSlotExp = kSmallSlotCnt + 1;
constexpr int kSmallSlotDrop = kSmallSlotExp + 1;
constexpr int kSmallVals = kSmallSlotDrop + 1;
static_assert(kSmallRoutes == 4 * kSmallKeyBatch * kSmallThreads, "the small path loads its ids in 1 or 4 batches");
static_assert(kSmallVals <= kSmallThreads, "one thread sums each counted value");

template <bool QUANT, int NB>
__global__ __launch_bounds__(kSmallThreads) void k_dispatch_small(
    const v4u* __restrict__ x, const int32_t* __restrict__ ids, const uint8_t* __restrict__ mask, int mask_per_route,
    v4u* __restrict__ expand_x, int8_t* __restrict__ expand_q, float* __restrict__ dyn_scale,
    int32_t* __restrict__ assist, int32_t* __restrict__ ep_recv, int64_t* __restrict__ expert_nums,
    int32_t* __restrict__ row_idx, const float* __restrict__ scales_in, float* __restrict__ scales_out,
    mdc_device_status* __restrict__ status, int W, int d, int BS, int K, int E, int L, int64_t A, int nvec,
    int n_ids) {
  __shared__ int part_s[kSmallThreads / 64][kSmallVals];   // per-wavefront counts
  __shared__ int tkey_s[MDC_MAX_TOPK];   // keys of this token's routes
  __shared__ int row_s[MDC_MAX_TOPK];
  __shared__ float amax_s[kSmallThreads / 64];
  const int tid = threadIdx.x;
  const int lane = tid & 63, wave = tid >> 6;
  const int tok = blockIdx.x;   // s * BS + t
  const int G = gridDim.x;      // W * BS
  const int s = tok / BS, t = tok - s * BS;
  const int n = W * BS * K;
  const int nc = L * W;
  const int per_src = BS * K;

  // Route ids and mask flags of all NB batches are loaded first, then this
  // token's own K ids (lane k of each wavefront loads route k), then the
  // token's row: straight-line code, so the counting below overlaps the row
  // loads.
  // Indices past the end are clamped, not skipped, and without a mask the
  // mask loads read the first route id's bytes and are ignored, so that the
  // loads are unconditional.
  constexpr int kB = kSmallKeyBatch * NB;
  int ev[kB];
  uint8_t mv[kB];
  const uint8_t* mptr = mask != nullptr ? mask : reinterpret_cast<const uint8_t*>(ids);
  const int mmul = mask == nullptr ? 0 : 1;
  const int mdiv = mask_per_route ? 1 : K;
#pragma unroll
  for (int j = 0; j < kB; ++j) ev[j] = ids[min(tid + j * kSmallThreads, n - 1)];
#pragma unroll
  for (int j = 0; j < kB; ++j) mv[j] = mptr[(min(tid + j * kSmallThreads, n - 1) / mdiv) * mmul];
  // lane k < K of every wavefront: route k of this token
  const int ftk = tok * K + min(lane, K - 1);
  const int tev = ids[ftk];
  const uint8_t tmv = mptr[(ftk / mdiv) * mmul];

  // (clamped as well: vectors past the row's end are never stored, and the
  // quantiser skips them).  The scheduling barriers keep every id and mask
  // load ahead of the row loads.
  const v4u* xr = x + (int64_t)tok * nvec;
  v4u cache[kSmallRowVec];
  __builtin_amdgcn_sched_barrier(0);
#pragma unroll
  for (int u = 0; u < kSmallRowVec; ++u) cache[u] = xr[min(tid + u * kSmallThreads, nvec - 1)];
  __builtin_amdgcn_sched_barrier(0);

  // key: local expert of an active route sent to d, else -1.  Conditions are
  // combined with bitwise operators: no branch for the compiler to sink an id
  // or mask load into (its wait would then also wait for the row loads).
  auto key_of = [&](int e, uint8_t m) {
    const int q = e - d * L;
    const bool ok = ((mask == nullptr) | (m != 0)) & (e >= 0) & (e < E) & (q >= 0) & (q < L);
    return ok ? q : -1;
  };
  // ck: (key, f) of route f as one unsigned number, key * 2^13 + f (f <
  // kSmallRoutes = 2^13), all ones for routes not sent here; "key below e,
  // or key e and route before g" is then ck < e * 2^13 + g
  static_assert(kSmallRoutes <= (1 << 13), "route index must fit 13 bits");
  unsigned ck[kB];
  bool drop[kB];   // active routes with ids outside [0, n_ids): dropped, counted by workgroup 0
#pragma unroll
  for (int j = 0; j < kB; ++j) {
    const int f = tid + j * kSmallThreads;
    const int q = key_of(ev[j], mv[j]);
    ck[j] = (f < n) & (q >= 0) ? ((unsigned)q << 13) | (unsigned)f : ~0u;
    drop[j] = (f < n) & ((mask == nullptr) | (mv[j] != 0)) & ((ev[j] < 0) | (ev[j] >= n_ids));
  }
  // (lanes >= K hold route K - 1's key and are never read: no select for
  // the compiler to turn into a branch around the loads)
  const int tk = key_of(tev, tmv);
  if (wave == 0 && lane < MDC_MAX_TOPK) tkey_s[lane] = tk;
  // routes of this wavefront's ids with lo <= ck < hi
  auto count = [&](unsigned lo, unsigned hi) {
    int c = 0;
#pragma unroll
    for (int j = 0; j < kB; ++j) c += (int)__popcll(__ballot((ck[j] >= lo) & (ck[j] < hi)));
    return c;
  };

  const int rounds = (nc + G - 1) / G;
  for (int r = 0; r < rounds; ++r) {
    if (r == 0) {
      // lane k collects the count of route k, then one store per lane
      int mine = 0;
#pragma unroll 1
      for (int k = 0; k < K; ++k) {
        const int kq = __builtin_amdgcn_readlane(tk, k);
        if (kq >= 0) {
          const int c = count(0u, ((unsigned)kq << 13) + (unsigned)(tok * K + k));
          mine = lane == k ? c : mine;
        }
      }
      if (lane < K) part_s[wave][lane] = mine;
      if (tok == 0) {
        int dc = 0;
#pragma unroll
        for (int j = 0; j < kB; ++j) dc += (int)__popcll(__ballot(drop[j]));
        if (lane == 0) part_s[wave][kSmallSlotDrop] = dc;
      }
    }
    const int ic = r * G + tok, ie = r * G + G - 1 - tok;
    if (ic < nc) {
      const int le = ic / W, lim = (ic - le * W + 1) * per_src;
      const int c = count(0u, ((unsigned)le << 13) + (unsigned)lim);   // (lim may be 2^13)
      if (lane == 0) part_s[wave][kSmallSlotCnt] = c;
    }
    if (ie < L) {
      const int c = count((unsigned)ie << 13, (unsigned)(ie + 1) << 13);
      if (lane == 0) part_s[wave][kSmallSlotExp] = c;
    }
    __syncthreads();
    if (tid < kSmallVals) {
      const int v = tid;
      const bool used = v < kSmallSlotCnt ? (r == 0 && v < K)
                        : v == kSmallSlotCnt ? ic < nc
                        : v == kSmallSlotExp ? ie < L
                        : (r == 0 && tok == 0);
      int sum = 0;
      if (used)
#pragma unroll
        for (int w = 0; w < kSmallThreads / 64; ++w) sum += part_s[w][v];
      if (v < kSmallSlotCnt) {
        if (used) {
          // this token's route k = v
          const int f = tok * K + v;
          int row = -1;
          if (tkey_s[v] >= 0) {
            row = sum < A ? sum : -1;
            row_idx[f] = row;
            if (row >= 0) {
              int32_t* a = assist + (int64_t)row * 3;
              a[0] = s;
              a[1] = t;
              a[2] = v;
              if (scales_out != nullptr) scales_out[row] = scales_in[f];
            }
          }
          row_s[v] = row;
        }
      } else if (v == kSmallSlotCnt) {
        if (used) {
          ep_recv[ic] = sum;   // inclusive ([TL] GetCumSum)
          if (ic == nc - 1) {
            // every route sent here
            const int64_t over = (int64_t)sum - A;
            status->overflow_rows = over > 0 ? (int32_t)over : 0;
            status->wait_timeouts = 0;
            status->reserved = 0;
          }
        }
      } else if (v == kSmallSlotExp) {
        if (used) expert_nums[ie] = (int64_t)sum;
      } else if (used) {
        status->dropped_ids = sum;
      }
    }
    __syncthreads();   // row_s is visible; part_s is free for the next round
  }
  bool any = false;
  for (int k = 0; k < K; ++k) any |= row_s[k] >= 0;
  if (!any) return;

  if (!QUANT) {
    for (int k = 0; k < K; ++k) {
      const int row = row_s[k];
      if (row < 0) continue;
      v4u* dst = expand_x + (int64_t)row * nvec;
#pragma unroll
      for (int u = 0; u < kSmallRowVec; ++u) {
        const int i = tid + u * kSmallThreads;
        if (i < nvec) dst[i] = cache[u];
      }
    }
  } else {
    // per-row int8 quantisation decided in fp32, as k_dispatch_gather_q
    float amax = 0.f;
#pragma unroll
    for (int u = 0; u < kSmallRowVec; ++u)
      if (tid + u * kSmallThreads < nvec)
#pragma unroll
        for (int w = 0; w < 4; ++w) amax = fmaxf(amax, fmaxf(fabsf(bf16_lo(cache[u][w])), fabsf(bf16_hi(cache[u][w]))));
#pragma unroll
    for (int o = 32; o >= 1; o >>= 1) amax = fmaxf(amax, __shfl_xor(amax, o, 64));
    if (lane == 0) amax_s[wave] = amax;
    __syncthreads();
#pragma unroll
    for (int w = 0; w < kSmallThreads / 64; ++w) amax = fmaxf(amax, amax_s[w]);
    const float inv = amax > 0.f ? 127.0f / amax : 0.f;
    const float scale = amax / 127.0f;
    if (tid < K && row_s[tid] >= 0) dyn_scale[row_s[tid]] = scale;
#pragma unroll
    for (int u = 0; u < kSmallRowVec; ++u) {
      const int i = tid + u * kSmallThreads;
      if (i >= nvec) continue;
      uint64_t packed = 0;
#pragma unroll
      for (int w = 0; w < 4; ++w) {
        const float a = fminf(fmaxf(rintf(bf16_lo(cache[u][w]) * inv), -127.f), 127.f);
        const float b = fminf(fmaxf(rintf(bf16_hi(cache[u][w]) * inv), -127.f), 127.f);
        packed |= (uint64_t)(uint8_t)(int8_t)(int)a << (16 * w);
        packed |= (uint64_t)(uint8_t)(int8_t)(int)b << (16 * w + 8);
      }
      for (int k = 0; k < K; ++k) {
        const int row = row_s[k];
        if (row >= 0) reinterpret_cast<uint64_t*>(expand_q + (int64_t)row * nvec * 8)[i] = packed;
      }
    }
  }
}

// Empty batch: every count is zero, and so is the status block.
__global__ __launch_bounds__(64) void k_zero_counts(int32_t* __restrict__ ep_recv, int64_t* __restrict__ expert_nums,
                                                    mdc_device_status* __restrict__ status, int L, int W) {
  for (int i = threadIdx.x; i < L * W; i += 64) ep_recv[i] = 0;
  for (int i = threadIdx.x; i < L; i += 64) expert_nums[i] = 0;
  if (threadIdx.x == 0) *status = mdc_device_status{0, 0, 0, 0};
}

// ---------------------------------------------------------------------------
// a6: combine.  One wavefront per (token t of rank r, column tile).
// ---------------------------------------------------------------------------
struct CombineTables {
  const v4u* y[MDC_MAX_COMBINE_WORLD];
  const int32_t* assist[MDC_MAX_COMBINE_WORLD];
  const int32_t* counts[MDC_MAX_COMBINE_WORLD];
  const float* esc[MDC_MAX_COMBINE_WORLD];   // expand_scales per rank (all NULL without the table)
};

// With performance_info, every combine wavefront records (start, end, ranks
// read) with the constant-rate real-time clock; k_combine_perf turns them
// into per-rank waits.
struct CombineRecord {
  uint64_t t0, t1, ranks;
};


// Route (r, t, k) is present when the token is active, 0 <= e < E, and row
// idx[t][k] of destination j = e / L is below min(count_j, A) and holds the
// triplet (r, t, k).  The prologue is two load levels: (ids, row index,
// scale, mask, pointer tables) then (count_j, triplet); every address is
// kept inside its buffer so the loads can be issued without branches.
template <int KMAX, int V, bool SHARED, bool TIMED>
__global__ __launch_bounds__(64 * MDC_COMBINE_WAVES) void k_combine(
    CombineTables tabs, const int32_t* __restrict__ row_idx, const int32_t* __restrict__ ids,
    const float* __restrict__ scales, const uint8_t* __restrict__ mask,
    const v4u* __restrict__ shared, const v4u* __restrict__ ori, v4u* __restrict__ out,
    CombineRecord* __restrict__ rec, int r, int W, int K, int E, int L, int64_t A, int nvec, int ntiles,
    unsigned n_items, int mask_per_route, int Z, int C, int has_esc) {
  const unsigned item = blockIdx.x * MDC_COMBINE_WAVES + (threadIdx.x >> 6);
  if (item >= n_items) return;
  const uint64_t t_start = TIMED ? __builtin_amdgcn_s_memrealtime() : 0;
  const int t = (int)(item / (unsigned)ntiles);
  const int tile = (int)(item - (unsigned)t * (unsigned)ntiles);
  const int lane = threadIdx.x & 63;
  const int kk = lane < K ? lane : 0;
  const int64_t rt = (int64_t)t * K + kk;

  // First load level, all in flight together: the per-lane pointer tables
  // (from the kernel arguments), then the route's id, row index, scale and
  // mask flag.  Without a mask the flag load reads the id's first byte and
  // is ignored, so that the load carries no branch.
  const int tl = lane < W ? lane : 0;
  const uint64_t yb = (uint64_t)tabs.y[tl];
  const uint64_t ab = (uint64_t)tabs.assist[tl];
  const uint64_t cb = (uint64_t)tabs.counts[tl];
  const int e = ids[rt];
  const int row = row_idx[rt];
  const float sc_route = scales[rt];
  const uint8_t mflag = mask != nullptr ? mask[mask_per_route ? rt : (int64_t)t]
                                        : *reinterpret_cast<const uint8_t*>(ids + rt);
  const bool act = (mask == nullptr) || (mflag != 0);

  const bool valid = (lane < K) && act && e >= 0 && e < E && A > 0;
  const int j = valid ? e / L : 0;
  const bool inrange = row >= 0 && row < A;
  const int64_t rowc = inrange ? row : 0;
  const uint64_t yj = shfl64(yb, j);
  const uint64_t aj = shfl64(ab, j);
  const uint64_t cj = shfl64(cb, j);

  bool ok = false;
  float sc = sc_route;
  if (A > 0) {
    const int32_t total = load_i32(cj + ((uint64_t)L * W - 1) * 4);
    const uint64_t a = aj + (uint64_t)rowc * 12;
    const int a0 = load_i32(a), a1 = load_i32(a + 4), a2 = load_i32(a + 8);
    if (has_esc) {   // the weight that travelled with the row (expand_scales of rank j)
      const uint64_t ej = shfl64((uint64_t)tabs.esc[tl], j);
      const float w = __builtin_bit_cast(float, load_i32(ej + (uint64_t)rowc * 4));
      if (valid) sc = w;
    }
    ok = valid && inrange && row < total && a0 == r && a1 == t && a2 == lane;
  }
  v4u* orow = out + (int64_t)t * nvec;
  // Zero experts [E, E+Z) and copy experts [E+Z, E+Z+C) are present without a
  // dispatched row: output 0 or the token's own row ori[t].
  const bool special = (lane < K) && act && e >= E && e - E < Z + C;
  const bool is_zero = special && e - E < Z;
  uint64_t yrow = yj + (uint64_t)rowc * (uint64_t)nvec * sizeof(v4u);
  if (special && !is_zero) yrow = (uint64_t)(ori + (int64_t)t * nvec);
  ok = ok || special;
  const uint64_t has = __ballot(ok);
  const uint64_t zero_lanes = __ballot(is_zero);
  const int np = __popcll(has);
  // A zero expert's slot is loaded and then replaced by zero: it reads a row
  // this wavefront loads anyway (the first present non-zero route's, else the
  // shared row), so the discarded load is served from cache, not HBM.
  const uint64_t srow = (uint64_t)(shared + (int64_t)t * nvec);
  const uint64_t nz = has & ~zero_lanes;
  const uint64_t alias = nz ? readlane64(yrow, __ffsll((unsigned long long)nz) - 1) : (SHARED ? srow : (uint64_t)orow);
  if (is_zero) yrow = alias;
  const int base = tile * 64 * V + lane;

  if (np == 0) {
    const v4u z = {0u, 0u, 0u, 0u};
#pragma unroll
    for (int u = 0; u < V; ++u) {
      const int idx = base + u * 64;
      if (idx < nvec) store_v4<MDC_COMBINE_NT_STORES != 0>(orow + idx, z);
    }
    if (TIMED && lane == 0) rec[item] = CombineRecord{t_start, t_start, 0};
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
    if (TIMED && u == V - 1) {
      // every row load has returned (its values are in acc): this wavefront's
      // arrival time for the ranks it read
      uint64_t ranks = (ok && !special) ? (1ull << j) : 0ull;
#pragma unroll
      for (int o2 = 32; o2 >= 1; o2 >>= 1) {
        const unsigned lo = __shfl_xor((unsigned)ranks, o2, 64), hi = __shfl_xor((unsigned)(ranks >> 32), o2, 64);
        ranks |= ((uint64_t)hi << 32) | lo;
      }
      const uint64_t t_end = __builtin_amdgcn_s_memrealtime();
      if (lane == 0) rec[item] = CombineRecord{t_start, t_end, ranks};
    }
    if (idx < nvec) store_v4<MDC_COMBINE_NT_STORES != 0>(orow + idx, o);
  }
}

// performance_info[j] += the wait for rank j's data: from the earliest
// wavefront start to the latest arrival of a row read from rank j, in whole
// microseconds rounded up (at least 1 for a rank that sent rows); ranks no
// row was read from are left unchanged.  One workgroup.
__global__ __launch_bounds__(1024) void k_combine_perf(const CombineRecord* __restrict__ rec, unsigned n_items,
                                                       int W, int64_t* __restrict__ perf, int64_t ticks_per_us) {
  __shared__ unsigned long long end_s[MDC_MAX_COMBINE_WORLD];
  __shared__ unsigned long long start_s[1024 / 64];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  if (tid < MDC_MAX_COMBINE_WORLD) end_s[tid] = 0ull;
  __syncthreads();
  unsigned long long t0 = ~0ull;
  for (unsigned i = tid; i < n_items; i += 1024) {
    const CombineRecord c = rec[i];
    t0 = c.t0 < t0 ? c.t0 : t0;
    uint64_t m = c.ranks;
    while (m) {
      const int jj = __ffsll((unsigned long long)m) - 1;
      m &= m - 1;
      atomicMax(&end_s[jj], (unsigned long long)c.t1);
    }
  }
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) {
    const unsigned long long v = ((unsigned long long)(unsigned)__shfl_xor((unsigned)(t0 >> 32), o, 64) << 32) |
                                 (unsigned)__shfl_xor((unsigned)t0, o, 64);
    t0 = v < t0 ? v : t0;
  }
  if (lane == 0) start_s[wave] = t0;
  __syncthreads();
  if (tid < W) {
    unsigned long long start = ~0ull;
    for (int w = 0; w < 1024 / 64; ++w) start = start_s[w] < start ? start_s[w] : start;
    const unsigned long long e = end_s[tid];
    if (e != 0ull) {
      const int64_t ticks = e > start ? (int64_t)(e - start) : 0;
      const int64_t us = (ticks + ticks_per_us - 1) / ticks_per_us;
      perf[tid] += us > 0 ? us : 1;
    }
  }
}

// ---------------------------------------------------------------------------
// Host side
// ---------------------------------------------------------------------------


mdc_status layout_impl(const DispatchPlan& p, const int32_t* ids, const uint8_t* mask, char* ws, hipStream_t st) {
  int32_t* P = reinterpret_cast<int32_t*>(ws + p.off_p);
  int32_t* cnt = reinterpret_cast<int32_t*>(ws + p.off_cnt);
  int32_t* drop = reinterpret_cast<int32_t*>(ws + p.off_drop);
  if (p.G == 0) return MDC_OK;
  (void)hipGetLastError();
  const size_t lds = (size_t)(p.rank_threads / 64 + 1) * p.L * sizeof(int32_t);
  hipLaunchKernelGGL(k_route_rank, dim3(p.G, p.W), dim3(p.rank_threads), lds, st,
                     ids, mask, P, cnt, drop, p.BS, p.K, p.E, p.L, p.d, p.W, p.TPG, p.G, p.mask_per_route, p.n_ids);
  return launched();
}

mdc_status gather_impl(const DispatchPlan& p, const void* x, const GatherMeta& m, void* expand_x, hipStream_t st) {
  (void)hipGetLastError();
  const int64_t tokens = (int64_t)p.W * p.BS;
  if (tokens == 0) {
    // nothing routed: zero the counts and the status block
    hipLaunchKernelGGL(k_zero_counts, dim3(1), dim3(64), 0, st, m.ep_recv, m.expert_nums, m.status, p.L, p.W);
    return launched();
  }
  // tiles of vpl vectors per lane (at most kGatherVec), and for vpl >= 5
  // also small tiles of kGatherSmallVec vectors per lane
  const int ntiles_big = (p.nvec + 64 * kGatherVec - 1) / (64 * kGatherVec);
  const int vpl = (p.nvec + 64 * ntiles_big - 1) / (64 * ntiles_big);
  const bool adaptive = vpl >= 5;   // the cases below that launch with VS = kGatherSmallVec < V
  const int ntiles = adaptive ? (p.nvec + 64 * kGatherSmallVec - 1) / (64 * kGatherSmallVec) : ntiles_big;
  const unsigned n_items = (unsigned)(tokens * ntiles);
  const dim3 grid((n_items + MDC_GATHER_WAVES - 1) / MDC_GATHER_WAVES), block(64 * MDC_GATHER_WAVES);
#define MDC_LAUNCH_GATHER(V, VS)                                                                              \
  hipLaunchKernelGGL((k_dispatch_gather<V, VS>), grid, block, 0, st, static_cast<const v4u*>(x), m,            \
                     static_cast<v4u*>(expand_x), p.BS, p.K, p.L, p.W, p.TPG, p.G, p.A, p.nvec, ntiles, n_items)
  switch (vpl) {
    case 1: MDC_LAUNCH_GATHER(1, 1); break;
    case 2: MDC_LAUNCH_GATHER(2, 2); break;
    case 3: MDC_LAUNCH_GATHER(3, 3); break;
    case 4: MDC_LAUNCH_GATHER(4, 4); break;
    case 5: MDC_LAUNCH_GATHER(5, kGatherSmallVec); break;
    case 6: MDC_LAUNCH_GATHER(6, kGatherSmallVec); break;
    case 7: MDC_LAUNCH_GATHER(7, kGatherSmallVec); break;
    default: MDC_LAUNCH_GATHER(8, kGatherSmallVec); break;
  }
#undef MDC_LAUNCH_GATHER
  return launched();
}

mdc_status gather_q_impl(const DispatchPlan& p, const void* x, const GatherMeta& m, int8_t* expand_q, float* dyn_scale,
                         hipStream_t st) {
  (void)hipGetLastError();
  const int64_t tokens = (int64_t)p.W * p.BS;
  if (tokens == 0) {
    hipLaunchKernelGGL(k_zero_counts, dim3(1), dim3(64), 0, st, m.ep_recv, m.expert_nums, m.status, p.L, p.W);
    return launched();
  }
  const int vpl = (p.nvec + 63) / 64;
#define MDC_LAUNCH_GQ(V)                                                                                          \
  hipLaunchKernelGGL(k_dispatch_gather_q<V>, dim3((unsigned)tokens), dim3(64), 0, st, static_cast<const v4u*>(x), \
                     m, expand_q, dyn_scale, p.BS, p.K, p.L, p.W, p.TPG, p.G, p.A, p.nvec)
  if (vpl <= 4) MDC_LAUNCH_GQ(4);
  else if (vpl <= 8) MDC_LAUNCH_GQ(8);
  else if (vpl <= 12) MDC_LAUNCH_GQ(12);
  else MDC_LAUNCH_GQ(16);
#undef MDC_LAUNCH_GQ
  return launched();
}

// Decode-size batches: the one-shot entry points (mdc_dispatch,
// mdc_dispatch_quant) run the whole dispatch as one launch of
// k_dispatch_small instead of the rank and gather kernels.  The split-stage
// entry points always take the two-kernel path (the gather stage does not
// see the ids).
bool small_path(const DispatchPlan& p) {
  const int64_t routes = (int64_t)p.W * p.BS * p.K;
  return routes > 0 && routes <= kSmallRoutes &&
         (int64_t)p.L * p.W <= (int64_t)kSmallMaxRounds * p.W * p.BS &&
         (int64_t)p.W * p.BS * routes <= kSmallRereads && p.nvec <= kSmallRowVec * kSmallThreads;
}

template <bool QUANT>
mdc_status small_impl(const DispatchPlan& p, const void* x, const int32_t* ids, const uint8_t* mask, void* expand_x,
                      int8_t* expand_q, float* dyn_scale, const GatherMeta& m, hipStream_t st) {
  (void)hipGetLastError();
  const bool one_batch = (int64_t)p.W * p.BS * p.K <= kSmallKeyBatch * kSmallThreads;
  auto kern = one_batch ? k_dispatch_small<QUANT, 1> : k_dispatch_small<QUANT, 4>;
  hipLaunchKernelGGL(kern, dim3((unsigned)(p.W * p.BS)), dim3(kSmallThreads), 0, st,
                     static_cast<const v4u*>(x), ids, mask, p.mask_per_route, static_cast<v4u*>(expand_x), expand_q,
                     dyn_scale, m.assist, m.ep_recv, m.expert_nums, m.row_idx, m.scales_in, m.scales_out, m.status,
                     p.W, p.d, p.BS, p.K, p.E, p.L, p.A, p.nvec, p.n_ids);
  return launched();
}

// Pointer checks of the gather stage (shared by the four dispatch entry points
// that place rows).  `rows` is expand_x or expand_q.

// Combine tiles: 64 * kCombineVec vectors per lane for K <= 8, one vector
// per lane otherwise.
int combine_tiles(int nvec, int K) {
  const int v = K <= 8 ? kCombineVec : 1;
  return (nvec + 64 * v - 1) / (64 * v);
}

// Workspace of mdc_combine: one CombineRecord per wavefront, used only with
// performance_info.
size_t combine_workspace_bytes(const mdc_shape* sh) {
  const size_t items = (size_t)sh->bs * combine_tiles(sh->hidden / 8, sh->topk);
  return round_up(items * sizeof(CombineRecord), 256);
}

template <int KMAX, int V, bool SHARED, bool TIMED>
void launch_combine(const CombineTables& tabs, const int32_t* row_idx, const int32_t* ids, const float* scales,
                    const uint8_t* mask, const v4u* sh, const v4u* ori, v4u* out, CombineRecord* rec,
                    const mdc_shape* shape, int ntiles, unsigned n_items, int has_esc, hipStream_t s) {
  const int W = shape->world;
  const dim3 grid((n_items + MDC_COMBINE_WAVES - 1) / MDC_COMBINE_WAVES), block(64 * MDC_COMBINE_WAVES);
  hipLaunchKernelGGL((k_combine<KMAX, V, SHARED, TIMED>), grid, block, 0, s, tabs, row_idx, ids, scales, mask, sh,
                     ori, out, rec, shape->rank, W, shape->topk, shape->num_experts, shape->num_experts / W,
                     (int64_t)shape->capacity, shape->hidden / 8, ntiles, n_items, shape->mask_per_route,
                     shape->zero_experts, shape->copy_experts, has_esc);
}

template <int KMAX, int V, bool TIMED>
void launch_combine_s(bool shared, const CombineTables& tabs, const int32_t* row_idx, const int32_t* ids,
                      const float* scales, const uint8_t* mask, const v4u* sh, const v4u* ori, v4u* out,
                      CombineRecord* rec, const mdc_shape* shape, int ntiles, unsigned n_items, int has_esc,
                      hipStream_t s) {
  if (shared)
    launch_combine<KMAX, V, true, TIMED>(tabs, row_idx, ids, scales, mask, sh, ori, out, rec, shape, ntiles, n_items,
                                         has_esc, s);
  else
    launch_combine<KMAX, V, false, TIMED>(tabs, row_idx, ids, scales, mask, sh, ori, out, rec, shape, ntiles, n_items,
                                          has_esc, s);
}

mdc_status combine_impl(const mdc_shape* shape, const void* const* expand_x, const int32_t* const* assist_info,
                        const int32_t* const* ep_recv_counts, const int32_t* expanded_row_idx,
                        const int32_t* expert_ids, const float* expert_scales, const uint8_t* x_active_mask,
                        const float* const* expand_scales, const void* shared_expert_x, const void* ori_x,
                        int64_t* perf, void* x_out, void* workspace, size_t workspace_bytes, hipStream_t s) {
  mdc_status st = check_shape(shape);
  if (st != MDC_OK) return st;
  const int W = shape->world;
  if (W > MDC_MAX_COMBINE_WORLD) return MDC_ERR_UNSUPPORTED;
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
    if (shape->capacity > 0 && expand_scales != nullptr && expand_scales[j] == nullptr) return MDC_ERR_NULLPTR;
    if (!aligned16(expand_x[j])) return MDC_ERR_INVALID;
    tabs.y[j] = static_cast<const v4u*>(expand_x[j]);
    tabs.assist[j] = assist_info[j];
    tabs.counts[j] = ep_recv_counts[j];
    tabs.esc[j] = expand_scales != nullptr ? expand_scales[j] : nullptr;
  }
  if (shape->copy_experts > 0 && ori_x == nullptr) return MDC_ERR_NULLPTR;
  if (!aligned16(shared_expert_x) || !aligned16(x_out) || !aligned16(ori_x)) return MDC_ERR_INVALID;
  CombineRecord* rec = nullptr;
  int64_t ticks_per_us = 100;
  if (perf != nullptr) {
    if (workspace == nullptr) return MDC_ERR_NULLPTR;
    if (workspace_bytes < combine_workspace_bytes(shape)) return MDC_ERR_WORKSPACE;
    rec = static_cast<CombineRecord*>(workspace);
    int dev = 0, khz = 0;
    if (hipGetDevice(&dev) != hipSuccess || hipDeviceGetAttribute(&khz, hipDeviceAttributeWallClockRate, dev) !=
                                                hipSuccess || khz < 1000)
      return MDC_ERR_HIP;
    ticks_per_us = khz / 1000;
  }
  const int K = shape->topk;
  const int nvec = shape->hidden / 8;
  const v4u* sh = static_cast<const v4u*>(shared_expert_x);
  v4u* out = static_cast<v4u*>(x_out);
  const v4u* ori = static_cast<const v4u*>(ori_x);
  const int has_esc = expand_scales != nullptr && shape->capacity > 0 ? 1 : 0;
  const int ntiles = combine_tiles(nvec, K);
  const unsigned n_items = (unsigned)((int64_t)BS * ntiles);
  const bool shared = sh != nullptr;
  (void)hipGetLastError();
  if (K <= 8) {
    if (perf)
      launch_combine_s<8, kCombineVec, true>(shared, tabs, expanded_row_idx, expert_ids, expert_scales, x_active_mask,
                                             sh, ori, out, rec, shape, ntiles, n_items, has_esc, s);
    else
      launch_combine_s<8, kCombineVec, false>(shared, tabs, expanded_row_idx, expert_ids, expert_scales,
                                              x_active_mask, sh, ori, out, rec, shape, ntiles, n_items, has_esc, s);
  } else {
    if (perf)
      launch_combine_s<16, 1, true>(shared, tabs, expanded_row_idx, expert_ids, expert_scales, x_active_mask, sh, ori,
                                    out, rec, shape, ntiles, n_items, has_esc, s);
    else
      launch_combine_s<16, 1, false>(shared, tabs, expanded_row_idx, expert_ids, expert_scales, x_active_mask, sh,
                                     ori, out, rec, shape, ntiles, n_items, has_esc, s);
  }
  if (perf != nullptr) {
    st = launched();
    if (st != MDC_OK) return st;
    hipLaunchKernelGGL(k_combine_perf, dim3(1), dim3(1024), 0, s, rec, n_items, W, perf, ticks_per_us);
  }
  return launched();
}

// Device address of this device's scratch array, looked up once per device
// (hipGetSymbolAddress with that device current) and kept; NULL if the lookup
// fails.
constexpr int kNoAllocMaxDevices = 64;
std::mutex g_scratch_mu;
void* g_scratch_ptr[kNoAllocMaxDevices] = {};

void* noalloc_scratch() {
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kNoAllocMaxDevices) return nullptr;
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (g_scratch_ptr[dev] == nullptr) {
    void* ptr = nullptr;
    if (hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch)) != hipSuccess || ptr == nullptr) return nullptr;
    g_scratch_ptr[dev] = ptr;
  }
  return g_scratch_ptr[dev];
}

}  // namespace

extern "C" {

const char* mdc_status_string(mdc_status status) {
  switch (status) {
    case MDC_OK: return "MDC_OK";
    case MDC_ERR_NULLPTR: return "MDC_ERR_NULLPTR: a required pointer is NULL";
    case MDC_ERR_INVALID: return "MDC_ERR_INVALID: misaligned tensor or shape fields that do not describe a problem";
    case MDC_ERR_UNSUPPORTED: return "MDC_ERR_UNSUPPORTED: a value outside the range this library supports";
    case MDC_ERR_WORKSPACE: return "MDC_ERR_WORKSPACE: workspace smaller than the size query returned";
    case MDC_ERR_HIP: return "MDC_ERR_HIP: a HIP kernel launch failed";
  }
  return "unknown mdc_status";
}

int32_t mdc_abi_version(void) { return MDC_ABI_VERSION; }

mdc_status mdc_dispatch_workspace(const mdc_shape* shape, size_t* bytes) {
  if (bytes == nullptr) return MDC_ERR_NULLPTR;
  mdc_status st = check_shape(shape);
  if (st != MDC_OK) return st;
  const DispatchPlan p = make_plan(shape);
  if ((st = check_plan(p)) != MDC_OK) return st;
  *bytes = p.bytes;
  return MDC_OK;
}

mdc_status mdc_dispatch_workspace_size(const mdc_shape* shape, size_t* bytes) {
  return mdc_dispatch_workspace(shape, bytes);
}

mdc_status mdc_dispatch_layout(const mdc_shape* shape, const int32_t* expert_ids, const uint8_t* x_active_mask,
                               void* workspace, size_t workspace_bytes, void* stream) {
  mdc_status st = check_shape(shape);
  if (st != MDC_OK) return st;
  const DispatchPlan p = make_plan(shape);
  if ((st = check_plan(p)) != MDC_OK) return st;
  if (workspace == nullptr) return MDC_ERR_NULLPTR;
  if (p.BS > 0 && expert_ids == nullptr) return MDC_ERR_NULLPTR;
  if (workspace_bytes < p.bytes) return MDC_ERR_WORKSPACE;
  return layout_impl(p, expert_ids, x_active_mask, static_cast<char*>(workspace), static_cast<hipStream_t>(stream));
}

mdc_status mdc_dispatch_gather(const mdc_shape* shape, const void* x, const float* expert_scales, void* expand_x,
                               int32_t* assist_info, int32_t* ep_recv_counts, int64_t* expert_token_nums,
                               int32_t* expanded_row_idx, float* expand_scales, void* workspace,
                               size_t workspace_bytes, void* stream) {
  mdc_status st = check_shape(shape);
  if (st != MDC_OK) return st;
  const DispatchPlan p = make_plan(shape);
  if ((st = check_plan(p)) != MDC_OK) return st;
  st = check_gather_args(p, x, expand_x, nullptr, false, assist_info, ep_recv_counts, expert_token_nums,
                         expanded_row_idx, expert_scales, expand_scales, workspace, workspace_bytes);
  if (st != MDC_OK) return st;
  char* ws = static_cast<char*>(workspace);
  const GatherMeta m = make_meta(p, ws, expert_scales, expand_scales, assist_info, ep_recv_counts,
                                 expert_token_nums, expanded_row_idx);
  return gather_impl(p, x, m, expand_x, static_cast<hipStream_t>(stream));
}

mdc_status mdc_dispatch(const mdc_shape* shape, const void* x, const int32_t* expert_ids,
                        const uint8_t* x_active_mask, const float* expert_scales, void* expand_x,
                        int32_t* assist_info, int32_t* ep_recv_counts, int64_t* expert_token_nums,
                        int32_t* expanded_row_idx, float* expand_scales, void* workspace, size_t workspace_bytes,
                        void* stream) {
  mdc_status st = check_shape(shape);
  if (st != MDC_OK) return st;
  const DispatchPlan p = make_plan(shape);
  if ((st = check_plan(p)) != MDC_OK) return st;
  if (p.BS > 0 && expert_ids == nullptr) return MDC_ERR_NULLPTR;
  st = check_gather_args(p, x, expand_x, nullptr, false, assist_info, ep_recv_counts, expert_token_nums,
                         expanded_row_idx, expert_scales, expand_scales, workspace, workspace_bytes);
  if (st != MDC_OK) return st;
  char* ws = static_cast<char*>(workspace);
  hipStream_t s = static_cast<hipStream_t>(stream);
  const GatherMeta m = make_meta(p, ws, expert_scales, expand_scales, assist_info, ep_recv_counts,
                                 expert_token_nums, expanded_row_idx);
  if (small_path(p)) return small_impl<false>(p, x, expert_ids, x_active_mask, expand_x, nullptr, nullptr, m, s);
  st = layout_impl(p, expert_ids, x_active_mask, ws, s);
  if (st != MDC_OK) return st;
  return gather_impl(p, x, m, expand_x, s);
}

mdc_status mdc_dispatch_noalloc(const mdc_shape* shape, const void* x, const int32_t* expert_ids,
                                const uint8_t* x_active_mask, const float* expert_scales, void* expand_x,
                                int32_t* assist_info, int32_t* ep_recv_counts, int64_t* expert_token_nums,
                                int32_t* expanded_row_idx, float* expand_scales, void* stream) {
  mdc_status st = check_shape(shape);
  if (st != MDC_OK) return st;
  const DispatchPlan p = make_plan(shape);
  if ((st = check_plan(p)) != MDC_OK) return st;
  if (p.bytes > (size_t)MDC_NOALLOC_SCRATCH_BYTES) return MDC_ERR_UNSUPPORTED;
  void* ws = noalloc_scratch();
  if (ws == nullptr) return MDC_ERR_HIP;
  // every workspace region the dispatch reads is written earlier in the same
  // call, so the scratch needs no clearing between calls
  return mdc_dispatch(shape, x, expert_ids, x_active_mask, expert_scales, expand_x, assist_info, ep_recv_counts,
                      expert_token_nums, expanded_row_idx, expand_scales, ws, (size_t)MDC_NOALLOC_SCRATCH_BYTES,
                      stream);
}

mdc_status mdc_dispatch_quant_gather(const mdc_shape* shape, const void* x, const float* expert_scales,
                                     int8_t* expand_q, float* dynamic_scales, int32_t* assist_info,
                                     int32_t* ep_recv_counts, int64_t* expert_token_nums, int32_t* expanded_row_idx,
                                     float* expand_scales, void* workspace, size_t workspace_bytes, void* stream) {
  mdc_status st = check_shape(shape);
  if (st != MDC_OK) return st;
  const DispatchPlan p = make_plan(shape);
  if ((st = check_plan(p)) != MDC_OK) return st;
  st = check_gather_args(p, x, expand_q, dynamic_scales, true, assist_info, ep_recv_counts, expert_token_nums,
                         expanded_row_idx, expert_scales, expand_scales, workspace, workspace_bytes);
  if (st != MDC_OK) return st;
  char* ws = static_cast<char*>(workspace);
  const GatherMeta m = make_meta(p, ws, expert_scales, expand_scales, assist_info, ep_recv_counts,
                                 expert_token_nums, expanded_row_idx);
  return gather_q_impl(p, x, m, expand_q, dynamic_scales, static_cast<hipStream_t>(stream));
}

mdc_status mdc_dispatch_quant(const mdc_shape* shape, const void* x, const int32_t* expert_ids,
                              const uint8_t* x_active_mask, const float* expert_scales, int8_t* expand_q,
                              float* dynamic_scales, int32_t* assist_info, int32_t* ep_recv_counts,
                              int64_t* expert_token_nums, int32_t* expanded_row_idx, float* expand_scales,
                              void* workspace, size_t workspace_bytes, void* stream) {
  mdc_status st = check_shape(shape);
  if (st != MDC_OK) return st;
  const DispatchPlan p = make_plan(shape);
  if ((st = check_plan(p)) != MDC_OK) return st;
  if (p.BS > 0 && expert_ids == nullptr) return MDC_ERR_NULLPTR;
  st = check_gather_args(p, x, expand_q, dynamic_scales, true, assist_info, ep_recv_counts, expert_token_nums,
                         expanded_row_idx, expert_scales, expand_scales, workspace, workspace_bytes);
  if (st != MDC_OK) return st;
  char* ws = static_cast<char*>(workspace);
  hipStream_t s = static_cast<hipStream_t>(stream);
  const GatherMeta m = make_meta(p, ws, expert_scales, expand_scales, assist_info, ep_recv_counts,
                                 expert_token_nums, expanded_row_idx);
  if (small_path(p)) return small_impl<true>(p, x, expert_ids, x_active_mask, nullptr, expand_q, dynamic_scales, m, s);
  st = layout_impl(p, expert_ids, x_active_mask, ws, s);
  if (st != MDC_OK) return st;
  return gather_q_impl(p, x, m, expand_q, dynamic_scales, s);
}

mdc_status mdc_combine_workspace(const mdc_shape* shape, size_t* bytes) {
  if (bytes == nullptr) return MDC_ERR_NULLPTR;
  const mdc_status st = check_shape(shape);
  if (st != MDC_OK) return st;
  *bytes = combine_workspace_bytes(shape);
  return MDC_OK;
}

mdc_status mdc_combine_workspace_size(const mdc_shape* shape, size_t* bytes) {
  return mdc_combine_workspace(shape, bytes);
}

mdc_status mdc_combine(const mdc_shape* shape, const void* const* expand_x, const int32_t* const* assist_info,
                       const int32_t* const* ep_recv_counts, const int32_t* expanded_row_idx,
                       const int32_t* expert_ids, const float* expert_scales, const uint8_t* x_active_mask,
                       const float* const* expand_scales, const void* shared_expert_x, const void* ori_x,
                       int64_t* performance_info, void* x_out, void* workspace, size_t workspace_bytes,
                       void* stream) {
  return combine_impl(shape, expand_x, assist_info, ep_recv_counts, expanded_row_idx, expert_ids, expert_scales,
                      x_active_mask, expand_scales, shared_expert_x, ori_x, performance_info, x_out, workspace,
                      workspace_bytes, static_cast<hipStream_t>(stream));
}

}  // extern "C"
