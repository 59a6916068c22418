// Route layout shared by the dispatch kernels and the pipelined dispatch +
// FFN: rank-group geometry, the group-counter order, the dispatch workspace,
// route placement and the per-row int8 quantisation of dispatched rows.
// Included after mdc_common.h by the kernel sources that need it.
#pragma once

#include "mdc_common.h"

namespace {

// Routes per rank group: 1024 (one step of a 1024-thread rank workgroup)
// measured 0.9 us faster per share step than 2048; 512 makes every gather
// wavefront scan 8 counter chunks, and 4096 halves the rank kernel's width.
#ifndef MDC_GROUP_ROUTES
#define MDC_GROUP_ROUTES 1024
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

// Rows of up to 64 * kQuantRowVec 16-byte vectors (H <= 8192) are quantised
// from registers, one wavefront per row.
constexpr int kQuantRowVec = 16;

// Pointers the gather kernels share beyond the rows themselves.
struct GatherMeta {
  const int32_t* P;           // packed (local expert, rank) per route
  const int32_t* cnt;         // group counters (transposed chunks)
  const int32_t* drop;        // dropped ids per rank group
  mdc_device_status* status;  // the workspace's status block
  const float* scales_in;     // [W][BS][K] route weights, or NULL
  float* scales_out;          // [A] expand_scales, or NULL
  int32_t* assist;
  int32_t* ep_recv;
  int64_t* expert_nums;
  int32_t* row_idx;
};

// Tile-0 work of a route placed at `row`: inverse-index entry, triplet and
// the weight that travels with the row.
__device__ __forceinline__ void place_route(const GatherMeta& m, int64_t g, int K, int s, int t, int lane, int row) {
  m.row_idx[g * K + lane] = row;
  if (row >= 0) {
    int32_t* a = m.assist + (int64_t)row * 3;
    a[0] = s;
    a[1] = t;
    a[2] = lane;
    if (m.scales_out != nullptr) m.scales_out[row] = m.scales_in[g * K + lane];
  }
}

// Per-row int8 quantisation of one bf16 row held by a wavefront (lane l
// holds vectors l + 64 u, u < VPL; vectors past the row are zero):
// scale = amax / 127 and codes clamp(rint(v * (127 / amax)), -127, 127),
// decided in fp32 ([CV4] dynamic quantisation of the communicated rows;
// [PTO] FrontReorder: quantised rows with a per-token scale).  qv[u] packs
// the 8 codes of vector u.
template <int VPL>
__device__ __forceinline__ float quant_row(const v4u (&v)[VPL], uint64_t (&qv)[VPL]) {
  float amax = 0.f;
#pragma unroll
  for (int u = 0; u < VPL; ++u)
#pragma unroll
    for (int w = 0; w < 4; ++w) amax = fmaxf(amax, fmaxf(fabsf(bf16_lo(v[u][w])), fabsf(bf16_hi(v[u][w]))));
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) amax = fmaxf(amax, __shfl_xor(amax, o, 64));
  const float inv = amax > 0.f ? 127.0f / amax : 0.f;
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
  return amax / 127.0f;
}

// ---------------------------------------------------------------------------
// Host side
// ---------------------------------------------------------------------------
struct DispatchPlan {
  int W, d, BS, H, K, E, L, TPG, G, nvec, rank_threads, mask_per_route, n_ids;
  int64_t A;
  size_t off_drop, off_p, off_cnt, off_base, bytes;
};

// Workspace: [status block][drop: W*G int32][P: W*BS*K int32][group counters]
// [group bases: L*W*G + 1 int32, written and read by the pipelined
// dispatch + FFN only].
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
  p.n_ids = sh->num_experts + sh->zero_experts + sh->copy_experts;
  p.TPG = kGroupRoutes / p.K;
  p.G = (p.BS + p.TPG - 1) / p.TPG;
  p.nvec = p.H / 8;
  // wave_cnt[nw][L] + carry[L] must fit in LDS: 16 wavefronts up to L = 512, 4 beyond
  p.rank_threads = p.L <= 512 ? 1024 : 256;
  const size_t routes = (size_t)p.W * p.BS * p.K;
  const size_t counters = round_up((size_t)p.L * p.W * p.G, kScanChunk);
  p.off_drop = MDC_STATUS_BYTES;
  p.off_p = p.off_drop + round_up((size_t)p.W * p.G * 4, 256);
  p.off_cnt = p.off_p + round_up(routes * 4, 256);
  p.off_base = p.off_cnt + round_up(counters * 4, 256);
  p.bytes = p.off_base + round_up(((size_t)p.L * p.W * p.G + 1) * 4, 256);
  return p;
}

// Group counters (and their bases, one more) are indexed in 32 bits.
mdc_status check_plan(const DispatchPlan& p) {
  return (int64_t)p.L * p.W * p.G + kScanChunk > INT32_MAX ? MDC_ERR_UNSUPPORTED : MDC_OK;
}

GatherMeta make_meta(const DispatchPlan& p, char* ws, const float* scales_in, float* scales_out, int32_t* assist,
                     int32_t* ep_recv, int64_t* expert_nums, int32_t* row_idx) {
  return GatherMeta{reinterpret_cast<const int32_t*>(ws + p.off_p), reinterpret_cast<const int32_t*>(ws + p.off_cnt),
                    reinterpret_cast<const int32_t*>(ws + p.off_drop), reinterpret_cast<mdc_device_status*>(ws),
                    scales_in, scales_out, assist, ep_recv, expert_nums, row_idx};
}

mdc_status check_gather_args(const DispatchPlan& p, const void* x, const void* rows, const float* dyn_scale,
                             bool quant, int32_t* assist, int32_t* ep_recv, int64_t* expert_nums, int32_t* row_idx,
                             const float* scales_in, float* scales_out, const void* ws, size_t ws_bytes) {
  if (quant && p.nvec > 64 * kQuantRowVec) return MDC_ERR_UNSUPPORTED;
  if (ws == nullptr || ep_recv == nullptr || expert_nums == nullptr) return MDC_ERR_NULLPTR;
  if (p.BS > 0 && (x == nullptr || row_idx == nullptr)) return MDC_ERR_NULLPTR;
  if (p.BS > 0 && p.A > 0 && (rows == nullptr || assist == nullptr || (quant && dyn_scale == nullptr)))
    return MDC_ERR_NULLPTR;
  if (p.BS > 0 && scales_out != nullptr && scales_in == nullptr) return MDC_ERR_NULLPTR;
  if (!aligned16(x) || !aligned16(rows)) return MDC_ERR_INVALID;
  if (ws_bytes < p.bytes) return MDC_ERR_WORKSPACE;
  return MDC_OK;
}

}  // namespace
