// libmdc: grouped int8 expert FFN of the MoE hot path for AMD Instinct MI355X
// (gfx950): mdc_ffn, mdc_ffn_quant_input, and mdc_dispatch_ffn (the quantised
// dispatch and the FFN as one pipeline).
//
// Source: "PTO MegaMoE Dispatch + Combine Fusion Example", GMM1 / SwiGLU /
// GMM2 stages and the per-token dynamic quantisation between them; Overall
// Architecture and Dispatch Stage for the pipeline.

#include "mdc_route.h"

namespace {

// ---------------------------------------------------------------------------
// a7: grouped int8 expert FFN ([PTO] GMM1 / SwiGLU / GMM2 stages).
//
// Per local expert e, on its expert-major rows of expand_x:
//   q1, s1 = per-row int8 quantisation of x (amax / 127, round half even)
//   h      = (q1 . W1[e]^T) * s1[row] * w1s[e][n]          (int32 MFMA accumulate)
//   g      = silu(h[:, j]) * h[:, j + N/2],  j < N/2        (fused in GMM1's epilogue)
//   q2, s2 = per-row int8 quantisation of g (per m-tile, once its GMM1 tiles are done)
//   y      = bf16((q2 . W2[e]^T) * s2[row] * w2s[e][h])
// The GEMMs use v_mfma_i32_32x32x32_i8 on 256-token x 256-weight-row tiles
// (GMM1: 128 gate + 128 up weight rows per tile so gate and up land in the
// same lanes), eight wavefronts (two per SIMD) each holding a 128 x 64 int32
// accumulator block in registers, k staged 128 bytes deep through two LDS
// arrays (a tile's first stage through registers, the others by direct
// global -> LDS loads); the output tile leaves through LDS as whole rows.  In
// the stream-ordered GEMMs an expert's tail of at most 32 rows per full m-tile
// rides along with its full m-tiles as a ninth 32-row token block instead of
// streaming the expert's weights once more in an m-tile of its own.  By
// default GMM1, the quantisation of g and GMM2 run as three stream-ordered
// kernels, each GEMM persistent and loading its next tile's first k stage
// before the current tile's output stores; with MDC_FLAG_FFN_PIPELINE they run
// as one persistent kernel with ready counters between them (k_ffn_fused), and
// mdc_dispatch_ffn adds the dispatch of the rows to that kernel's queue.
// ---------------------------------------------------------------------------
typedef int v4i __attribute__((ext_vector_type(4)));
typedef unsigned int v2u __attribute__((ext_vector_type(2)));
typedef int v16i __attribute__((ext_vector_type(16)));

constexpr int kFfnBM = 256;        // token rows per tile
constexpr int kFfnBW = 256;        // weight rows per tile (GMM1: 128 gate + 128 up)
constexpr int kFfnBK = 128;        // k bytes per LDS stage
constexpr int kFfnThreads = 512;   // 8 wavefronts: 2 along tokens x 4 along weight rows
constexpr int kFfnStage = (kFfnBM + kFfnBW) * kFfnBK;   // bytes of one LDS stage
// An expert's tail of at most kFfnExtRows rows per full m-tile rides along
// with its full m-tiles (the stream-ordered GEMMs only): such an m-tile holds
// kFfnBM + up to kFfnExtRows token rows, the extra 32-row block of each k
// stage staged in an LDS array of its own (kFfnExtBytes, one per stage
// parity).
constexpr int kFfnExtRows = 32;
constexpr int kFfnExtBytes = kFfnExtRows * kFfnBK;
constexpr int kFfnOutAlign = 128;  // GMM output widths (N/2 and H) must be multiples of this

// Tile plan shared by both GEMMs.  Each local expert's rows (contiguous,
// expert-major, clipped at A) split into m-tiles of kFfnBM rows, the last
// one partial.  The table lists them in expert order and cuts each expert's
// run into chunks of at most kFfnChunkM consecutive m-tiles (sizes as equal
// as possible); the GEMM walks a chunk's tiles together (ffn_decode_tile),
// so an expert's partial m-tile runs beside its full ones and reads the
// weight tiles they bring into L2.  tiles[0].x = number of m-tiles;
// tiles[1 + m] = {expert, first row, expert's end row, (position in its
// chunk << 8) | chunk size}.  One workgroup of 1024 threads; L <= 2048 (two
// experts per thread).
constexpr int kFfnChunkM = 8;
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

// The fused kernel's synchronisation words (sync_words, stride = the
// table's capacity in m-tiles): [0] queue head, [1] unused, then done1,
// ready and rows_ready at [2 + i * stride, 2 + i * stride + MT) for
// i = 0, 1, 2, then emt[L] (first m-tile of each expert) and elo[L] (its
// first row).
struct FfnSyncLayout {
  int* w;
  int stride, L;
  __host__ __device__ int* next() const { return w; }
  __host__ __device__ int* done1() const { return w + 2; }
  __host__ __device__ int* ready() const { return w + 2 + stride; }
  __host__ __device__ int* rows_ready() const { return w + 2 + 2 * stride; }
  __host__ __device__ int* emt() const { return w + 2 + 3 * stride; }
  __host__ __device__ int* elo() const { return w + 2 + 3 * stride + L; }
  __host__ __device__ static size_t words(int stride, int L) { return 2 + 3 * (size_t)stride + 2 * (size_t)L; }
};

// Builds the tile plan from the expert counts c0, c1 of experts 2t and
// 2t + 1 (thread t; zero past L); with sw.w != NULL it also zeroes the
// fused kernel's synchronisation words and amax_bits for the rows in use
// and records each expert's first m-tile and first row.  Zeroes the
// workspace's status block.  Table entry 1 + m = {expert, first row, end
// row, chunk position << 8 | chunk size} of m-tile m.  Without sw.w (the
// stream-ordered GEMMs) an expert of n rows whose tail t = n % kFfnBM is at
// most kFfnExtRows per full m-tile has n / kFfnBM m-tiles, the first ones
// holding kFfnExtRows rows more each until the tail is placed: the tail
// rows then share their m-tiles' weight stages instead of streaming the
// expert's weights once more for a nearly empty m-tile.
__device__ void ffn_plan_body(int64_t c0, int64_t c1, int L, int64_t A, int4* __restrict__ tiles, FfnSyncLayout sw,
                              uint32_t* __restrict__ amax_bits, mdc_device_status* __restrict__ status,
                              int64_t* wsum) {
  const int tid = threadIdx.x;
  const int e0 = 2 * tid, e1 = 2 * tid + 1;
  int64_t total;
  const int64_t x0 = plan_scan_pair(c0, c1, wsum, total);   // first row of e0 (unclipped)
  const int64_t x1 = x0 + c0;
  const int lo0 = (int)min(x0, A), hi0 = (int)min(x0 + c0, A);
  const int lo1 = (int)min(x1, A), hi1 = (int)min(x1 + c1, A);
  const bool ext = sw.w == nullptr;
  // m-tiles of an expert with n rows (see above)
  auto mtiles = [&](int n) {
    const int f = n / kFfnBM, t = n - f * kFfnBM;
    return ext && f > 0 && t <= kFfnExtRows * f ? f : (n + kFfnBM - 1) / kFfnBM;
  };
  const int n0 = mtiles(hi0 - lo0), n1 = mtiles(hi1 - lo1);
  int64_t nm;
  const int p0 = (int)plan_scan_pair(n0, n1, wsum, nm);   // table slot of e0's first m-tile
  for (int h = 0; h < 2; ++h) {
    const int e = h ? e1 : e0, n = h ? n1 : n0, lo = h ? lo1 : lo0, hi = h ? hi1 : hi0;
    const int slot = h ? p0 + n0 : p0;
    const int tail = hi - lo - n * kFfnBM;   // > 0: rows riding along, kFfnExtRows per m-tile
    // chunks: nch of them, the first `big` with base + 1 m-tiles, the rest with base
    const int nch = (n + kFfnChunkM - 1) / kFfnChunkM;
    const int base = nch ? n / nch : 0, big = nch ? n % nch : 0;
    for (int j = 0; j < n; ++j) {
      int pos, size;
      if (j < big * (base + 1)) {
        pos = j % (base + 1);
        size = base + 1;
      } else {
        pos = (j - big * (base + 1)) % base;
        size = base;
      }
      const int r0 = lo + j * kFfnBM + (tail > 0 ? min(tail, kFfnExtRows * j) : 0);
      const int r1 = tail > 0 ? r0 + kFfnBM + min(kFfnExtRows, max(0, tail - kFfnExtRows * j)) : min(hi, r0 + kFfnBM);
      tiles[1 + slot + j] = int4{e, r0, r1, (pos << 8) | size};
    }
    if (sw.w != nullptr && e < L) {
      sw.emt()[e] = slot;
      sw.elo()[e] = lo;
    }
  }
  if (tid == 0) {
    tiles[0] = int4{(int)nm, 0, 0, 0};
    *status = mdc_device_status{0, 0, 0, 0};
  }
  if (sw.w != nullptr) {
    const int MT = (int)nm;
    if (tid < 2) sw.w[tid] = 0;
    for (int i = tid; i < MT; i += kPlanThreads) {
      sw.done1()[i] = 0;
      sw.ready()[i] = 0;
      sw.rows_ready()[i] = 0;
    }
    const int64_t rows = min(total, A);
    for (int64_t r = tid; r < rows; r += kPlanThreads) amax_bits[r] = 0u;
  }
}

__global__ __launch_bounds__(kPlanThreads) void k_ffn_plan(const int64_t* __restrict__ expert_nums, int L, int64_t A,
                                                           int4* __restrict__ tiles, FfnSyncLayout sw,
                                                           uint32_t* __restrict__ amax_bits,
                                                           mdc_device_status* __restrict__ status) {
  __shared__ int64_t wsum[kPlanThreads / 64 + 1];
  const int e0 = 2 * threadIdx.x, e1 = e0 + 1;
  const int64_t c0 = e0 < L ? expert_nums[e0] : 0, c1 = e1 < L ? expert_nums[e1] : 0;
  ffn_plan_body(c0, c1, L, A, tiles, sw, amax_bits, status, wsum);
}

// ---------------------------------------------------------------------------
// Pipelined dispatch + FFN (mdc_dispatch_ffn), launch 1 of 3.  One workgroup
// scans the group counters left by mdc_dispatch_layout once, in (le, s, g)
// order ([TL] GetCumSum; [PTO] FrontReorder publishes the prefix metadata
// once for every later stage): the exclusive prefix at a group is the first
// row of its routes (base), the inclusive prefix at (le, s, G - 1) is
// epRecvCounts[le*W + s], the difference across le's groups is
// expertTokenNums[le].  It fills the dispatch status block as the gather
// kernels do, then builds the FFN tile plan from the counts.
// ---------------------------------------------------------------------------
__global__ __launch_bounds__(kPlanThreads) void k_dfn_plan(
    const int32_t* __restrict__ cnt, const int32_t* __restrict__ drop, int32_t* __restrict__ base, int L, int W,
    int G, int64_t A, int32_t* __restrict__ ep_recv, int64_t* __restrict__ expert_nums,
    mdc_device_status* __restrict__ dstatus, int4* __restrict__ tiles, FfnSyncLayout sw,
    uint32_t* __restrict__ amax_bits, mdc_device_status* __restrict__ fstatus) {
  __shared__ int64_t wsum[kPlanThreads / 64 + 1];
  __shared__ int ecnt[2 * kPlanThreads];   // per-expert counts (L <= 2048)
  __shared__ int drop_s;
  const int tid = threadIdx.x;
  const int n = L * W * G;   // below 2^31 (host check)
  const int span = W * G;    // counters per expert
  constexpr int kPer = 4;    // consecutive counters per thread per chunk
  for (int e = tid; e < L; e += kPlanThreads) ecnt[e] = 0;
  if (tid == 0) drop_s = 0;
  int dropped = 0;
  for (int i = tid; i < span; i += kPlanThreads) dropped += drop[i];
  __syncthreads();
  if (dropped != 0) atomicAdd(&drop_s, dropped);
  int64_t carry = 0;
  for (int c0 = 0; c0 < n; c0 += kPlanThreads * kPer) {
    const int i0 = c0 + tid * kPer;
    int v[kPer];
    int64_t own = 0;
#pragma unroll
    for (int j = 0; j < kPer; ++j) {
      v[j] = i0 + j < n ? cnt[counter_slot(i0 + j)] : 0;
      own += v[j];
    }
    int64_t tot;
    int64_t run = carry + plan_scan_pair(own, 0, wsum, tot);
    // bases, epRecvCounts (inclusive prefix at each (le, s)'s last group) and
    // the per-expert sums, from the counters this thread holds
    int e_cur = -1, e_sum = 0;
#pragma unroll
    for (int j = 0; j < kPer; ++j) {
      const int i = i0 + j;
      if (i < n) {
        base[i] = (int32_t)run;
        if (i % G == G - 1) ep_recv[i / G] = (int32_t)(run + v[j]);
        const int e = i / span;
        if (e != e_cur) {
          if (e_sum != 0) atomicAdd(&ecnt[e_cur], e_sum);
          e_cur = e;
          e_sum = 0;
        }
        e_sum += v[j];
      }
      run += v[j];
    }
    if (e_sum != 0) atomicAdd(&ecnt[e_cur], e_sum);
    carry += tot;
  }
  if (tid == 0) base[n] = (int32_t)carry;
  if (G == 0)   // no tokens: no groups, every count is zero
    for (int i = tid; i < L * W; i += kPlanThreads) ep_recv[i] = 0;
  __syncthreads();
  const int e0 = 2 * tid, e1 = e0 + 1;
  const int64_t c0 = e0 < L ? ecnt[e0] : 0, c1 = e1 < L ? ecnt[e1] : 0;
  if (e0 < L) expert_nums[e0] = c0;
  if (e1 < L) expert_nums[e1] = c1;
  if (tid == 0) {
    const int64_t over = carry - A;
    *dstatus = mdc_device_status{drop_s, over > 0 ? (int32_t)over : 0, 0, 0};
  }
  ffn_plan_body(c0, c1, L, A, tiles, sw, amax_bits, fstatus, wsum);
}

// Launch 2 of 3: places every route sent here (one thread per route):
// row = base of its group + its rank, dropped past the capacity; writes the
// inverse index, the (source, token, k) triplet and the route's weight as
// the gather kernels' tile-0 work does.
__global__ __launch_bounds__(256) void k_dfn_route(GatherMeta m, const int32_t* __restrict__ base, int BS, int K,
                                                   int L, int W, int TPG, int G, int64_t A, int n_routes) {
  const int f = blockIdx.x * 256 + threadIdx.x;
  if (f >= n_routes) return;
  const int p = m.P[f];
  if (p < 0 || (p & 0xFFFF) >= L) return;
  const int g = f / K, k = f - g * K;
  const int s = g / BS, t = g - s * BS;
  const int64_t r = (int64_t)base[((p & 0xFFFF) * W + s) * G + t / TPG] + (p >> 16);
  place_route(m, g, K, s, t, k, r < A ? (int)r : -1);
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
// wavefront per row, rows [0, min(sum(expert_nums), A)) visited grid-stride.
// Rows of up to 64 * QV vectors stay in registers between the passes; with
// QV <= 8 each wavefront loads its next row before it quantises the current
// one (unconditional loads: vectors past the row's end reload its last
// vector and are neither counted nor stored).  Longer rows are streamed
// twice.
template <int QV>
__global__ __launch_bounds__(256) void k_ffn_quant_rows(
    const v4u* __restrict__ x, int8_t* __restrict__ q, float* __restrict__ scale,
    const int64_t* __restrict__ expert_nums, int L, int64_t A, int nvec) {
  constexpr bool kPrefetch = QV <= 8;
  const int lane = threadIdx.x & 63;
  const int64_t nw = (int64_t)gridDim.x * 4;
  // rows in use: sum of the expert counts, one load per lane and a
  // wavefront sum (a loop of dependent loads would open every wavefront
  // with L memory round trips)
  int64_t total = 0;
  for (int i = lane; i < L; i += 64) total += expert_nums[i];
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) {
    const unsigned lo = __shfl_xor((unsigned)(uint64_t)total, o, 64);
    const unsigned hi = __shfl_xor((unsigned)((uint64_t)total >> 32), o, 64);
    total += (int64_t)(((uint64_t)hi << 32) | lo);
  }
  const int64_t rows = total < A ? total : A;
  const bool cached = nvec <= 64 * QV;
  auto load_row = [&](int64_t row, auto& c) {   // c holds at least QV vectors
    const v4u* xr = x + row * nvec;
    if constexpr (kPrefetch) {
#pragma unroll
      for (int u = 0; u < QV; ++u) c[u] = xr[min(lane + 64 * u, nvec - 1)];
    } else {
      // (guarded loads keep one base address with immediate offsets)
#pragma unroll
      for (int u = 0; u < QV; ++u) {
        const int i = lane + 64 * u;
        c[u] = i < nvec ? xr[i] : v4u{0u, 0u, 0u, 0u};
      }
    }
  };
  auto quant8 = [](const v4u& v, float inv) {
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
  int64_t row = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6);
  if (row >= rows) return;
  v4u cache[QV], next[kPrefetch ? QV : 1];
  if (cached) load_row(row, cache);
  for (; row < rows; row += nw) {
    const v4u* xr = x + row * nvec;
    uint64_t* qr = reinterpret_cast<uint64_t*>(q + row * (int64_t)nvec * 8);
    if constexpr (kPrefetch) {
      if (cached) load_row(min(row + nw, rows - 1), next);
    }
    float amax = 0.f;
    if (cached) {
#pragma unroll
      for (int u = 0; u < QV; ++u)
        if (lane + 64 * u < nvec)
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
    if (cached) {
#pragma unroll
      for (int u = 0; u < QV; ++u) {
        const int i = lane + 64 * u;
        if (i < nvec) qr[i] = quant8(cache[u], inv);
      }
    } else {
      for (int i = lane; i < nvec; i += 64) qr[i] = quant8(xr[i], inv);
    }
    if (lane == 0) scale[row] = amax / 127.0f;
    if (cached) {
      if constexpr (kPrefetch) {
#pragma unroll
        for (int u = 0; u < QV; ++u) cache[u] = next[u];
      } else if (row + nw < rows) {
        load_row(row + nw, cache);
      }
    }
  }
}

// Launches the quantiser instance for rows of nvec vectors.
void launch_quant_rows(const v4u* x, int8_t* q, float* scale, const int64_t* expert_nums, int L, int64_t A, int nvec,
                       unsigned wgs, hipStream_t s) {
  if (nvec <= 64 * 4)
    hipLaunchKernelGGL(k_ffn_quant_rows<4>, dim3(wgs), dim3(256), 0, s, x, q, scale, expert_nums, L, A, nvec);
  else
    hipLaunchKernelGGL(k_ffn_quant_rows<16>, dim3(wgs), dim3(256), 0, s, x, q, scale, expert_nums, L, A, nvec);
}

// Buffer descriptors and offsets with which one thread stages one tile.
struct FfnStaging {
  __amdgpu_buffer_rsrc_t ra, rw;   // token rows, weight rows (range-checked)
  unsigned va, vw;                 // lane offsets of this thread's i = 0 rows
  unsigned whi;                    // extra weight offset of rows i >= 2 (GMM1: gate -> up)
  int K;
  int lds_off;                     // this thread's LDS byte offset for i = 0
};

// Stage 0 of a tile (k bytes 0 .. kFfnBK of this thread's staging rows)
// and the epilogue scale this thread loads, in registers.  A persistent
// kernel that knows its next tile loads them before the current tile's
// output stores: loads and stores retire in order, so a load issued after
// the stores would first wait for them to drain.
struct FfnStage0 {
  v4i sa[4], sw[4];
  float sc;
  float sc9;   // extended m-tiles: row scale of token row kFfnBM + t (threads t < kFfnExtRows)
};

// Loads k bytes k0 .. k0 + kFfnBK of this thread's staging rows (4 token
// rows and 4 weight rows, 16 bytes each) into registers.
template <bool COH>
__device__ __forceinline__ void ffn_stage_load(const FfnStaging& st, int k0, v4i (&sa)[4], v4i (&sw)[4]) {
  // COH: token rows are read with agent-coherent (sc1) loads: they were
  // written in the same launch by another workgroup, possibly on another XCD
  constexpr int kAux = COH ? 0x10 : 0;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    sa[i] = __builtin_amdgcn_raw_buffer_load_b128(st.ra, st.va + (unsigned)(64 * i * st.K), (unsigned)k0, kAux);
    sw[i] = __builtin_amdgcn_raw_buffer_load_b128(st.rw, st.vw + (unsigned)(64 * i * st.K) + (i >= 2 ? st.whi : 0u),
                                                  (unsigned)k0, 0);
  }
}

// The extra token rows kFfnBM .. + 32 of an extended m-tile, k bytes
// k0 .. k0 + kFfnBK, loaded global -> LDS directly into x (kFfnExtBytes):
// wavefront w < 4 loads rows kFfnBM + 8 w .. + 8 as one 1 KB block, lane l
// taking row kFfnBM + 8 w + l / 8 and LDS slot l % 8, which holds chunk
// (l % 8) ^ ((row / 2) & 7) (the swizzle of every staged row; (row / 2) & 7
// = (4 w + l / 16) & 7).  Rows past the tile read as zero.
__device__ __forceinline__ void ffn_stage_dma9(const FfnStaging& st, uint8_t* x, int k0) {
  typedef __attribute__((address_space(3))) void lds_void;
  const int lane = threadIdx.x & 63;
  const int wv = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  if (wv >= 4) return;
  const unsigned vo = (unsigned)((lane >> 3) * st.K) + (unsigned)(((lane & 7) ^ ((4 * wv + (lane >> 4)) & 7)) << 4);
  __builtin_amdgcn_raw_ptr_buffer_load_lds(st.ra, (lds_void*)(x + wv * 1024), 16, vo,
                                           (unsigned)k0 + (unsigned)((kFfnBM + 8 * wv) * st.K), 0, 0);
}

// The k loop of one tile (see ffn_tile).  The two k stages live in two LDS
// arrays, l0 (even stages) and l1 (odd stages).  Stage 0 comes through
// registers (loaded ahead by the persistent walk, or here), every later
// stage goes global -> LDS directly (buffer loads with the lds bit: no
// register round trip, no LDS write instructions): stage ks + 1 is loaded
// into the other array while stage ks is read, each wavefront waits for its
// own loads (vmcnt 0) before the barrier that ends the stage, and the next
// load into an array is issued only after that barrier.  Because the arrays
// are distinct objects, the compiler does not make reads of one wait for
// loads into the other.  Fragments of k substep q + 1 are read while the
// MFMAs of substep q run, and the last substep's MFMAs run after the stage
// barrier, beside the next stage's first fragment reads.  Scheduling groups
// (sched_group_barrier masks: 0x8 MFMA, 0x100 LDS read) interleave the
// fragment reads with the MFMAs.
//
// A direct load writes lane l's 16 bytes at the block base + 16 l: wavefront
// w loads 1 KB blocks 4w .. 4w + 3 of the token rows and of the weight rows
// (8 rows per block), lane l taking row 8 b + l / 8 and LDS slot l % 8, which
// holds chunk (l % 8) ^ ((row / 2) & 7) of the row: the layout the register
// path writes.
//
// NB = number of the wavefront's 32-row token blocks that hold valid rows:
// blocks past them stay zero, and their fragment reads and MFMAs are not
// issued (an expert's short last m-tile is cheap).  NB = 0 still stages and
// joins the barriers.
//
// X9: the m-tile is extended (NB = 4): the extra 32 token rows of even and
// odd stages sit in x0 and x1 (ffn_stage_dma9; stage 0's is issued with the
// stage 0 loads, before them, so it has landed when they have), and
// wavefront (wt, wn) also multiplies them by its weight block wt into acc9
// (GLU: wt = 0 gate, wt = 1 up rows of its quarter).
template <bool GLU, int NB, bool COH, bool X9 = false>
__device__ __forceinline__ void ffn_kloop(uint8_t* l0, uint8_t* l1, uint8_t* x0, uint8_t* x1, v16i (&acc)[2][4],
                                          v16i& acc9, const FfnStaging& st, int wt, int wn, const int (&fr)[4],
                                          const FfnStage0& s0, bool pre) {
  static_assert(!X9 || NB == 4, "an extended m-tile has all token blocks");
  constexpr int NCOLS = GLU ? kFfnBW / 2 : kFfnBW;
  constexpr int NR = NB > 0 ? NB + 2 + (X9 ? 1 : 0) : 0;   // fragment reads per k substep
  constexpr int NM = 2 * NB + (X9 ? 1 : 0);                // MFMAs per k substep
  constexpr int kAux = COH ? 0x10 : 0;      // token rows written in the same launch: agent-coherent loads
  typedef __attribute__((address_space(3))) void lds_void;
  const int lane = threadIdx.x & 63;
  const int wv = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  // LDS row of weight block j (32 rows) within the stage's weight tile
  auto wrow = [&](int j) {
    if (GLU) return j == 0 ? wn * 32 : NCOLS + wn * 32;
    return wn * 64 + 32 * j;
  };
  auto frags = [&](const uint8_t* sb, const uint8_t* sx, int q, v4i (&tf)[4], v4i (&wf)[2], v4i& t9) {
    if (NB == 0) return;
#pragma unroll
    for (int i = 0; i < NB; ++i) tf[i] = *reinterpret_cast<const v4i*>(sb + (wt * 128 + 32 * i) * kFfnBK + fr[q]);
#pragma unroll
    for (int j = 0; j < 2; ++j)
      wf[j] = *reinterpret_cast<const v4i*>(sb + kFfnBM * kFfnBK + wrow(j) * kFfnBK + fr[q]);
    if (X9) t9 = *reinterpret_cast<const v4i*>(sx + fr[q]);
  };
  auto mfmas = [&](const v4i (&tf)[4], const v4i (&wf)[2], const v4i& t9) {
#pragma unroll
    for (int i = 0; i < NB; ++i)
#pragma unroll
      for (int j = 0; j < 2; ++j) acc[j][i] = __builtin_amdgcn_mfma_i32_32x32x32_i8(wf[j], tf[i], acc[j][i], 0, 0, 0);
    if (X9) acc9 = __builtin_amdgcn_mfma_i32_32x32x32_i8(wt ? wf[1] : wf[0], t9, acc9, 0, 0, 0);
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
  // Direct-load offsets.  Block b = 4 wv + j holds rows 8 b + l / 8; the
  // lane part (row within the block, swizzled chunk) depends on j only
  // through j's parity ((row / 2) & 7 = (4 j + l / 16) & 7), and the block's
  // row offset (with GMM1's gate -> up jump for the weight rows of wavefronts
  // 4..7, blocks 16..31) is wavefront-uniform: it goes in the scalar offset.
  unsigned vo[2];
#pragma unroll
  for (int par = 0; par < 2; ++par)
    vo[par] = (unsigned)((lane >> 3) * st.K) + (unsigned)(((lane & 7) ^ ((4 * par + (lane >> 4)) & 7)) << 4);
  const unsigned whi_w = (GLU && wv >= 4) ? st.whi : 0u;
  auto dma = [&](uint8_t* buf, uint8_t* xbuf, int k0) {
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int blk = 4 * wv + j;
      const unsigned so = (unsigned)k0 + (unsigned)(8 * blk * st.K);
      __builtin_amdgcn_raw_ptr_buffer_load_lds(st.ra, (lds_void*)(buf + blk * 1024), 16, vo[j & 1], so, 0, kAux);
      __builtin_amdgcn_raw_ptr_buffer_load_lds(st.rw, (lds_void*)(buf + kFfnBM * kFfnBK + blk * 1024), 16, vo[j & 1],
                                               so + whi_w, 0, 0);
    }
    // extra token rows kFfnBM + 8 wv .. + 8 (block parity wv & 1)
    if (X9 && wv < 4)
      __builtin_amdgcn_raw_ptr_buffer_load_lds(st.ra, (lds_void*)(xbuf + wv * 1024), 16, vo[wv & 1],
                                               (unsigned)k0 + (unsigned)((kFfnBM + 8 * wv) * st.K), 0, kAux);
  };

  const int nk = st.K / kFfnBK;
  {
    // stage 0 through registers
    v4i sa[4], sw[4];
    if (pre) {
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        sa[i] = s0.sa[i];
        sw[i] = s0.sw[i];
      }
    } else {
      if (X9) ffn_stage_dma9(st, x0, 0);
      ffn_stage_load<COH>(st, 0, sa, sw);
    }
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      *reinterpret_cast<v4i*>(l0 + st.lds_off + 64 * i * kFfnBK) = sa[i];
      *reinterpret_cast<v4i*>(l0 + kFfnBM * kFfnBK + st.lds_off + 64 * i * kFfnBK) = sw[i];
    }
  }
  if (nk > 1) dma(l1, x1, kFfnBK);
  __syncthreads();
  v4i tf[4], wf[2], tg[4], wg[2], tf9, tg9;
  frags(l0, x0, 0, tf, wf, tf9);
  // one stage: substeps 0..2 from cur, then (after the barrier) the load of
  // stage ks + 2 into cur and substep 3's MFMAs beside stage ks + 1's first reads
  auto stage = [&](uint8_t* cur, uint8_t* nxt, uint8_t* ccur, uint8_t* cnxt, int ks) {
    frags(cur, ccur, 1, tg, wg, tg9);
    mfmas(tf, wf, tf9);
    interleave_reads();
    frags(cur, ccur, 2, tf, wf, tf9);
    mfmas(tg, wg, tg9);
    interleave_reads();
    frags(cur, ccur, 3, tg, wg, tg9);
    mfmas(tf, wf, tf9);
    interleave_reads();
    __builtin_amdgcn_s_waitcnt(0x0F70);   // vmcnt(0): this wavefront's loads into nxt have landed
    __syncthreads();
    if (ks + 2 < nk) dma(cur, ccur, (ks + 2) * kFfnBK);
    frags(nxt, cnxt, 0, tf, wf, tf9);   // (after the last stage: read, never used)
    mfmas(tg, wg, tg9);
    interleave_reads();
  };
  for (int ks = 0; ks < nk; ks += 2) {
    stage(l0, l1, x0, x1, ks);
    if (ks + 1 < nk) stage(l1, l0, x1, x0, ks + 1);
  }
}

// Grouped GEMM tiles, C = A . W[e]^T with A int8 [rows][K] (token rows of
// expert e) and W int8 [L][Nw][K].  GLU = true (GMM1): each tile pairs 128
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
// Epilogue: scales come from LDS; the wavefronts write their bf16 outputs
// into the (now free) LDS as [256 rows][tile columns], 16-byte units XOR-
// swizzled by row, then every thread stores 16 bytes of a whole row.
//
// Tiles: T = (m-tiles of the plan) x (output columns / tile columns).  The
// launches hold one workgroup per CU.  k_ffn_gemm: workgroup b walks tiles
// i*G + (b % 8)*(G/8) + b / 8; hardware places workgroup b on XCD b % 8, so
// each XCD walks a contiguous run of tiles, ordered by ffn_decode_tile in
// groups of up to 8 m-tiles of one expert x about 32 / (their number)
// n-tiles (m fastest) so the tiles an XCD runs together share A and W tiles
// in its L2.  k_ffn_fused takes the same order from an atomic queue.

// Operands of one grouped GEMM.
struct FfnGemm {
  const int8_t* a_src;      // [rows][K] int8 token rows, expert-major
  const float* row_scale;   // [rows]
  const int8_t* w;          // [L][Nw][K] int8
  const float* w_scale;     // [L][Nw]
  uint16_t* out;            // [rows][Nout] bf16
  int K, Nw, Nout;
};

// The kernel's LDS, shared by every tile it runs.
struct FfnSmem {
  uint8_t* l0;      // kFfnStage bytes: even k stages, then output rows 0..127
  uint8_t* l1;      // kFfnStage bytes: odd k stages, then output rows 128..255
  float* sc_row;    // [kFfnBM (+ kFfnExtRows)] row scales of the tile's token rows
  float* sc_col;    // [kFfnBW] weight-row scales (GMM1: 128 gate, then 128 up)
  uint8_t* x0;      // kFfnExtBytes each: the extra rows of even / odd k stages
  uint8_t* x1;      // (kernels whose plans hold extended m-tiles)
};

// Buffer descriptors and this thread's staging offsets for tile (ti, nt):
// token rows [row0, min(row_end, row0 + 256)) and weight rows [n0, Nw) of
// expert e (GMM1: up rows at Nw/2 + n0 + ...).  Thread t moves chunk t & 7
// of rows 64 i + t / 8 (i < 4) of both tiles; in LDS that chunk sits at
// slot (t & 7) ^ ((row / 2) & 7), and (row / 2) & 7 = (t / 16) & 7 for every
// i.  Weight rows relative to n0: i < 2 -> rows 64 i + t / 8 (GMM1: gate),
// i >= 2 -> GMM1: up rows Nw/2 + 64 (i - 2) + t / 8, GMM2: rows 64 i + t / 8.
template <bool GLU>
__device__ __forceinline__ FfnStaging ffn_staging(const FfnGemm& g, int4 ti, int nt) {
  constexpr int NCOLS = GLU ? kFfnBW / 2 : kFfnBW;
  const int tid = threadIdx.x;
  const int st_row = tid >> 3;
  const int st_chunk = tid & 7;
  const int st_lds = st_row * kFfnBK + ((st_chunk ^ ((tid >> 4) & 7)) << 4);
  const int K = g.K, Nw = g.Nw;
  const int e = __builtin_amdgcn_readfirstlane(ti.x);
  const int row0 = __builtin_amdgcn_readfirstlane(ti.y);
  const int row_end = __builtin_amdgcn_readfirstlane(ti.z);
  const int n0 = nt * NCOLS;
  const int rows_here = min(row_end - row0, kFfnBM + kFfnExtRows);   // (only extended m-tiles exceed kFfnBM)
  const __amdgpu_buffer_rsrc_t ra = __builtin_amdgcn_make_buffer_rsrc(
      const_cast<int8_t*>(g.a_src + (int64_t)row0 * K), (short)0, rows_here * K, 0x00020000);
  const __amdgpu_buffer_rsrc_t rw = __builtin_amdgcn_make_buffer_rsrc(
      const_cast<int8_t*>(g.w + ((int64_t)e * Nw + n0) * K), (short)0, (Nw - n0) * K, 0x00020000);
  const unsigned whi = GLU ? (unsigned)((Nw / 2 - NCOLS) * K) : 0u;
  const unsigned v0 = (unsigned)(st_row * K + st_chunk * 16);
  return FfnStaging{ra, rw, v0, v0, whi, K, st_lds};
}

// This thread's epilogue scale of tile (ti, nt): threads t < kFfnBM take
// the row scale of token row t, the others weight-row scale t - kFfnBM
// (GMM1: 128 gate rows, then the 128 matching up rows).
template <bool GLU, bool COH>
__device__ __forceinline__ float ffn_scale(const FfnGemm& g, int4 ti, int nt) {
  constexpr int NCOLS = GLU ? kFfnBW / 2 : kFfnBW;
  const int tid = threadIdx.x;
  const int e = __builtin_amdgcn_readfirstlane(ti.x);
  const int row0 = __builtin_amdgcn_readfirstlane(ti.y);
  const int row_end = __builtin_amdgcn_readfirstlane(ti.z);
  const int Nw = g.Nw, n0 = nt * NCOLS;
  if (tid < kFfnBM) {
    const float* rsp = g.row_scale + min(row0 + tid, row_end - 1);
    return COH ? __hip_atomic_load(rsp, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) : *rsp;
  }
  const int c = tid - kFfnBM;
  const int wr = GLU ? (c < NCOLS ? n0 + c : Nw / 2 + n0 + (c - NCOLS)) : min(n0 + c, Nw - 1);
  return g.w_scale[(int64_t)e * Nw + wr];
}

// One output tile: token rows [row0, min(row_end, row0 + 256)) of expert e
// (ti = {e, row0, row_end}) times n-tile nt.  GLU with amax_bits != NULL also
// folds max |g| of every stored row into amax_bits[row] (fp32 bits; g >= 0
// bit patterns order like the floats).  With have, cur already holds the
// tile's stage 0 and scale.  PF: once the accumulators are spent, next()
// (run by every thread) names the tile to load ahead, and nxt receives its
// stage 0 and scale when the returned pf is set (else this tile's own
// again, so that nxt is written on every call); cur is read before the k
// loop and nxt written after it, so nxt may be cur.  Returns what next()
// returned (PF) or pf = false.
struct FfnNext {
  bool pf;    // nxt holds stage 0 and scale of tile (ti, nt)
  int4 ti;
  int nt;
};

// EXT: the plan may hold extended m-tiles (up to kFfnBM + kFfnExtRows rows;
// the LDS stages then hold kFfnExtStage bytes); their extra rows are
// computed beside the others (ffn_kloop's X9) and leave through registers.
template <bool GLU, bool COH, bool PF, bool EXT, class NextF>
__device__ __forceinline__ FfnNext ffn_tile(const FfnGemm& g, int4 ti, int nt, const FfnSmem& sm,
                                            uint32_t* __restrict__ amax_bits, FfnStage0& cur, bool have,
                                            FfnStage0& nxt, NextF&& next) {
  constexpr int NCOLS = GLU ? kFfnBW / 2 : kFfnBW;   // output columns per tile
  constexpr int OU = NCOLS / 8;                      // 16-byte output units per tile row
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  // wavefront-uniform values are read into scalar registers (readfirstlane)
  const int wv = __builtin_amdgcn_readfirstlane(tid >> 6);
  // SIMD s runs wavefronts s and s + 4: one of each token half
  const int wt = wv >> 2;   // token half of the tile
  const int wn = wv & 3;    // weight-row quarter of the tile
  // fragment reads: lane l reads row l & 31, chunk 2 s + l / 32 (k substep s)
  int fr[4];
#pragma unroll
  for (int q = 0; q < 4; ++q) fr[q] = (lane & 31) * kFfnBK + (((2 * q + (lane >> 5)) ^ ((lane >> 1) & 7)) << 4);

  const int Nout = g.Nout;
  const int row0 = __builtin_amdgcn_readfirstlane(ti.y);
  const int row_end = __builtin_amdgcn_readfirstlane(ti.z);
  const int n0 = nt * NCOLS;
  const int rows_here = min(row_end - row0, kFfnBM);
  const bool x9 = EXT && row_end - row0 > kFfnBM;   // extended m-tile (uniform)
  const FfnStaging st = ffn_staging<GLU>(g, ti, nt);
  const float scv = have ? cur.sc : ffn_scale<GLU, COH>(g, ti, nt);
  // row scales of the extra token rows (extended m-tiles; threads < kFfnExtRows)
  const float sc9 = !x9 ? 0.f : have ? cur.sc9 : g.row_scale[min(row0 + kFfnBM + tid, row_end - 1)];
  __syncthreads();   // the previous tile is done with LDS
  // the epilogue's scales, read from LDS after the k loop's first barrier
  if (tid < kFfnBM) sm.sc_row[tid] = scv;
  else sm.sc_col[tid - kFfnBM] = scv;
  if (x9 && tid < kFfnExtRows) sm.sc_row[kFfnBM + tid] = sc9;

  // acc[j][i]: weight block j (32 rows), token block i (32 rows)
  v16i acc[2][4], acc9 = v16i{};
#pragma unroll
  for (int j = 0; j < 2; ++j)
#pragma unroll
    for (int i = 0; i < 4; ++i) acc[j][i] = v16i{};
  // 32-row token blocks of this wavefront's half that hold valid rows
  const int nblk = __builtin_amdgcn_readfirstlane(min(4, max(0, (rows_here - wt * 128 + 31) / 32)));
  if (EXT && x9) {
    ffn_kloop<GLU, 4, COH, EXT>(sm.l0, sm.l1, sm.x0, sm.x1, acc, acc9, st, wt, wn, fr, cur, have);
  } else {
    switch (nblk) {
      case 4: ffn_kloop<GLU, 4, COH>(sm.l0, sm.l1, sm.x0, sm.x1, acc, acc9, st, wt, wn, fr, cur, have); break;
      case 3: ffn_kloop<GLU, 3, COH>(sm.l0, sm.l1, sm.x0, sm.x1, acc, acc9, st, wt, wn, fr, cur, have); break;
      case 2: ffn_kloop<GLU, 2, COH>(sm.l0, sm.l1, sm.x0, sm.x1, acc, acc9, st, wt, wn, fr, cur, have); break;
      case 1: ffn_kloop<GLU, 1, COH>(sm.l0, sm.l1, sm.x0, sm.x1, acc, acc9, st, wt, wn, fr, cur, have); break;
      default: ffn_kloop<GLU, 0, COH>(sm.l0, sm.l1, sm.x0, sm.x1, acc, acc9, st, wt, wn, fr, cur, have); break;
    }
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
    const float rs = sm.sc_row[trow];
    uint8_t* orow = (wt ? sm.l1 : sm.l0) + (trow & 127) * (NCOLS * 2);
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
          const float hg = (float)acc[0][i][4 * q + jj] * rs * sm.sc_col[c + jj];
          const float hu = (float)acc[1][i][4 * q + jj] * rs * sm.sc_col[NCOLS + c + jj];
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
          for (int jj = 0; jj < 4; ++jj) v[jj] = (float)acc[j][i][4 * q + jj] * rs * sm.sc_col[c + jj];
          put(c, ffn_pack_bf16(v[0], v[1]), ffn_pack_bf16(v[2], v[3]));
        }
    }
  }
  // Extended m-tile: lane l holds token row kFfnBM + (l & 31) and, for run
  // q, columns cb + 8 q + cq .. + 3 of its weight block.  GLU: the up
  // values (wt = 1) go to LDS past the staged output rows, [wn][32 rows][36
  // floats] (padded rows), for the gate wavefront (wt = 0) of the same
  // quarter; the stream-ordered GEMMs, the only ones with extended m-tiles,
  // take no amax_bits.
  float* xup = reinterpret_cast<float*>(sm.l1 + 128 * NCOLS * 2) + wn * (32 * 36) + (lane & 31) * 36;
  const float rs9 = sm.sc_row[min(kFfnBM + (lane & 31), EXT ? kFfnBM + kFfnExtRows - 1 : kFfnBM - 1)];
  if (GLU && EXT && x9 && wt == 1) {
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      const int c = wn * 32 + 8 * q + cq;
      float4 hu;
      hu.x = (float)acc9[4 * q + 0] * rs9 * sm.sc_col[NCOLS + c + 0];
      hu.y = (float)acc9[4 * q + 1] * rs9 * sm.sc_col[NCOLS + c + 1];
      hu.z = (float)acc9[4 * q + 2] * rs9 * sm.sc_col[NCOLS + c + 2];
      hu.w = (float)acc9[4 * q + 3] * rs9 * sm.sc_col[NCOLS + c + 3];
      *reinterpret_cast<float4*>(xup + 8 * q + cq) = hu;
    }
  }
  // the accumulators are spent: load the next tile's stage 0 and scale now,
  // ahead of this tile's output stores
  const FfnNext nx = PF ? next() : FfnNext{false, ti, nt};
  if (PF) {
    const int4 pti = nx.pf ? nx.ti : ti;
    const int pnt = nx.pf ? nx.nt : nt;
    const FfnStaging pst = ffn_staging<GLU>(g, pti, pnt);
    // (an extended next tile's extra rows of stage 0 go to x0 first: they
    // have landed once the stage 0 registers have.  Only for a real next
    // tile, whose k loop waits for them: no direct load into LDS may be in
    // flight when the workgroup ends.)
    const bool px9 = EXT && nx.pf && pti.z - pti.y > kFfnBM;
    if (px9) ffn_stage_dma9(pst, sm.x0, 0);
    ffn_stage_load<COH>(pst, 0, nxt.sa, nxt.sw);
    nxt.sc = ffn_scale<GLU, COH>(g, pti, pnt);
    if (px9) nxt.sc9 = g.row_scale[min(pti.y + kFfnBM + tid, pti.z - 1)];
  }
  __syncthreads();
  if (EXT && x9 && (!GLU || wt == 0)) {
    // the extra rows leave from registers, 8 bytes (4 columns) per store
    const int row = row0 + kFfnBM + (lane & 31);
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      const int c = GLU ? wn * 32 + 8 * q + cq : wn * 64 + 32 * wt + 8 * q + cq;
      float v[4];
      if (GLU) {
        const float4 hu = *reinterpret_cast<const float4*>(xup + 8 * q + cq);
        const float hus[4] = {hu.x, hu.y, hu.z, hu.w};
#pragma unroll
        for (int jj = 0; jj < 4; ++jj) v[jj] = ffn_silu((float)acc9[4 * q + jj] * rs9 * sm.sc_col[c + jj]) * hus[jj];
      } else {
#pragma unroll
        for (int jj = 0; jj < 4; ++jj) v[jj] = (float)acc9[4 * q + jj] * rs9 * sm.sc_col[c + jj];
      }
      if (row < row_end && n0 + c < Nout)
        *reinterpret_cast<uint2*>(g.out + (int64_t)row * Nout + n0 + c) =
            uint2{ffn_pack_bf16(v[0], v[1]), ffn_pack_bf16(v[2], v[3])};
    }
  }
  const int u = tid % OU;
  const int col = n0 + u * 8;
#pragma unroll 4
  for (int rr = tid / OU; rr < kFfnBM; rr += kFfnThreads / OU) {
    const int row = row0 + rr;
    const v4u v = *reinterpret_cast<const v4u*>((rr < 128 ? sm.l0 : sm.l1) + (rr & 127) * (NCOLS * 2) +
                                                ((u ^ (rr % OU)) * 16));
    if (row < row_end && col < Nout) {
      // GMM2's y rows are stored non-temporal: the combine reads them once,
      // later, and the weights and token rows of the next GEMMs keep the
      // caches (GMM2 1% faster, and the combine and the next GMM1 gain too).
      // GMM1's g rows stay cached for the quantiser that reads them next.
      if (GLU) *reinterpret_cast<v4u*>(g.out + (int64_t)row * Nout + col) = v;
      else __builtin_nontemporal_store(v, reinterpret_cast<v4u*>(g.out + (int64_t)row * Nout + col));
    }
    if (GLU && amax_bits != nullptr) {
      // max |g| over this row's NCOLS columns: the OU threads of a row are
      // consecutive lanes of one wavefront
      float m = 0.f;
#pragma unroll
      for (int w = 0; w < 4; ++w) m = fmaxf(m, fmaxf(fabsf(bf16_lo(v[w])), fabsf(bf16_hi(v[w]))));
#pragma unroll
      for (int o = OU / 2; o >= 1; o >>= 1) m = fmaxf(m, __shfl_xor(m, o, 64));
      if (u == 0 && row < row_end) atomicMax(amax_bits + row, __float_as_uint(m));
    }
  }
  return nx;
}

// Tile t of a walk over T = MT x nn tiles -> (m-tile, n-tile).  The tiles
// of a chunk of h m-tiles (see the plan) are t in [m0 nn, (m0 + h) nn); they
// run in groups of h m-tiles x GN = 32 / h n-tiles, m fastest, so the about
// 32 tiles an XCD runs together share A and W tiles in its L2.
// All values are wavefront-uniform and below 2^31 (the host checks the
// tile count), so the divisions run in 32 bits on scalar registers.
template <typename Tab>
__device__ __forceinline__ void ffn_decode_tile(int t, int nn, const Tab& tab, int& mt, int& nt) {
  t = __builtin_amdgcn_readfirstlane(t);
  nn = __builtin_amdgcn_readfirstlane(nn);
  const int mrow = t / nn;
  const int w = __builtin_amdgcn_readfirstlane(tab.at(mrow).w);
  const int h = w & 255;
  const int m0 = mrow - (w >> 8);
  const int r = t - m0 * nn;
  const int gn = 32 / h;
  const int band = h * gn;
  const int ng = r / band;
  const int r2 = r - ng * band;
  const int q = r2 / h;
  mt = m0 + (r2 - q * h);
  nt = ng * gn + q;
}

// The m-tile table, read by the persistent kernels once per tile.  With
// TAB the kernel copies it into LDS at its start: a global read of a tile's
// entry would wait behind the previous tile's output stores (loads and
// stores retire in order), an LDS read does not.  The host takes TAB when
// the table fits (kFfnTabCache entries, kFfnTabCacheExt for the GEMMs whose
// LDS stages hold extended m-tiles); otherwise entries are read from global
// memory.
constexpr int kFfnTabCache = 1536;
constexpr int kFfnTabCacheExt = 1024;

template <bool TAB>
struct FfnTab {
  const int4* g;   // the plan's table (entry m at g[1 + m])
  int4* s;         // LDS copy (TAB)
  __device__ __forceinline__ int4 at(int m) const { return TAB ? s[m] : g[1 + m]; }
};

template <bool TAB, int CAP = kFfnTabCache>
__device__ __forceinline__ void ffn_cache_tab(const int4* __restrict__ tiles, int4* tab_s, int MT) {
  if (!TAB) return;
  const int n = min(MT, CAP);   // MT <= CAP whenever the host picks TAB
  for (int i = threadIdx.x; i < n; i += kFfnThreads) tab_s[i] = tiles[1 + i];
  __syncthreads();
}

// Persistent grouped GEMM over the plan's tiles (one workgroup per CU); the
// plan may hold extended m-tiles.
template <bool GLU, bool TAB>
__global__ __launch_bounds__(kFfnThreads) void k_ffn_gemm(FfnGemm g, const int4* __restrict__ tiles) {
  __shared__ __attribute__((aligned(16))) uint8_t lds0[kFfnStage];
  __shared__ __attribute__((aligned(16))) uint8_t lds1[kFfnStage];
  __shared__ __attribute__((aligned(16))) uint8_t ldx0[kFfnExtBytes];
  __shared__ __attribute__((aligned(16))) uint8_t ldx1[kFfnExtBytes];
  __shared__ float sc_row[kFfnBM + kFfnExtRows];
  __shared__ float sc_col[kFfnBW];
  __shared__ int4 tab_s[TAB ? kFfnTabCacheExt : 1];
  const FfnSmem sm{lds0, lds1, sc_row, sc_col, ldx0, ldx1};
  constexpr int NCOLS = GLU ? kFfnBW / 2 : kFfnBW;
  const int G = gridDim.x;
  const int nn = (g.Nout + NCOLS - 1) / NCOLS;
  const int MT = __builtin_amdgcn_readfirstlane(tiles[0].x);
  const int T = MT * nn;
  const int b = blockIdx.x;
  const int lin = (b % 8) * (G / 8) + b / 8;   // XCD-contiguous walk (G is a multiple of 8)
  ffn_cache_tab<TAB, kFfnTabCacheExt>(tiles, tab_s, MT);
  const FfnTab<TAB> tab{tiles, tab_s};
  int t = lin;
  if (t >= T) return;
  int mt, nt;
  ffn_decode_tile(t, nn, tab, mt, nt);
  int4 ti = tab.at(mt);
  FfnStage0 s0;
  const FfnStaging st0 = ffn_staging<GLU>(g, ti, nt);
  const bool x9 = ti.z - ti.y > kFfnBM;
  if (x9) ffn_stage_dma9(st0, ldx0, 0);
  ffn_stage_load<false>(st0, 0, s0.sa, s0.sw);
  s0.sc = ffn_scale<GLU, false>(g, ti, nt);
  if (x9) s0.sc9 = g.row_scale[min(ti.y + kFfnBM + (int)threadIdx.x, ti.z - 1)];
  for (;;) {
    // the next tile of this workgroup's walk; its stage 0 is loaded before
    // this tile's output stores
    const int tn = t + G;
    const bool has_next = tn < T;
    int mtn = mt, ntn = nt;
    if (has_next) ffn_decode_tile(tn, nn, tab, mtn, ntn);
    const int4 te = tab.at(mtn);
    const int4 tin = int4{__builtin_amdgcn_readfirstlane(te.x), __builtin_amdgcn_readfirstlane(te.y),
                          __builtin_amdgcn_readfirstlane(te.z), 0};
    ffn_tile<GLU, false, true, true>(g, ti, nt, sm, nullptr, s0, true, s0,
                                     [&]() { return FfnNext{has_next, tin, ntn}; });
    if (!has_next) break;
    t = tn;
    mt = mtn;
    nt = ntn;
    ti = tin;
  }
}

// Synchronisation words of the fused FFN kernel (workspace; the plan kernel
// zeroes them before every call).
struct FfnSync {
  int* next;              // work-queue head
  int* done1;             // [MT] GMM1 tiles finished per m-tile
  int* ready;             // [MT] 1 once the m-tile's g rows are quantised
  int* rows_ready;        // [MT] rows of the m-tile dispatched (pipelined dispatch only)
  uint32_t* amax_bits;    // [rows] max |g| per row (fp32 bits)
  mdc_device_status* status;   // wait_timeouts counts the waits that ran out of their bound
};

// A tile whose wait ran out does not read its inputs: its output tile is
// written as quiet NaN (GMM1: and its rows' max |g| as NaN, so that their
// quantised g and y follow), so that a silently wrong y cannot result.
// ncols: output columns per n-tile.
__device__ void ffn_poison_tile(const FfnGemm& g, int4 ti, int nt, int ncols, uint32_t* amax_bits) {
  const int row0 = ti.y, row_end = min(ti.z, ti.y + kFfnBM);
  const int n0 = nt * ncols, n1 = min(g.Nout, n0 + ncols);
  const int units = (n1 - n0) / 8;   // Nout is a multiple of 128
  const v4u nan = {0x7FC07FC0u, 0x7FC07FC0u, 0x7FC07FC0u, 0x7FC07FC0u};
  for (int i = threadIdx.x; i < (row_end - row0) * units; i += kFfnThreads) {
    const int r = row0 + i / units, c = n0 + (i % units) * 8;
    *reinterpret_cast<v4u*>(g.out + (int64_t)r * g.Nout + c) = nan;
  }
  if (amax_bits != nullptr)
    for (int r = row0 + (int)threadIdx.x; r < row_end; r += kFfnThreads) atomicMax(amax_bits + r, 0x7FC00000u);
}

// Waits (thread 0; the caller broadcasts the result) until *word >= need,
// polling with agent-coherent relaxed loads, at most spin_limit times.
// Returns true when the bound ran out, counted in the status block.
__device__ bool ffn_wait_at_least(const int* word, int need, int spin_limit, mdc_device_status* status) {
  int n = 0;
  while (__hip_atomic_load(word, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) < need) {
    if (++n >= spin_limit) {
      atomicAdd(&status->wait_timeouts, 1);
      return true;
    }
    __builtin_amdgcn_s_sleep(2);
  }
  return false;
}

// Makes every wavefront's global stores of the workgroup visible at agent
// scope before thread 0's next atomic: each wavefront waits for its own
// stores to complete (vmcnt 0), the barrier joins them, and thread 0 issues
// one agent-scope release (an L2 write-back).  Ends with a barrier.
__device__ __forceinline__ void ffn_publish_begin() {
  __builtin_amdgcn_s_waitcnt(0x0F70);   // vmcnt(0); expcnt, lgkmcnt untouched
  __syncthreads();
  if (threadIdx.x == 0) __builtin_amdgcn_fence(__ATOMIC_RELEASE, "agent");
}

// The pipelined dispatch's inputs to the fused kernel.
struct FfnDispatchIn {
  const v4u* x;            // [W][BS][H] bf16 source rows
  const int32_t* assist;   // [A][3] (source, token, k) of each row, placed by k_dfn_route
  int BS, nvec;
};

// Dispatch work of one queue item: rows [lo, hi) of one m-tile, each read
// from its source row (assist triplet), quantised per row (quant_row, as the
// quantised gather does) and written as int8 codes and a scale.  Wavefront w
// handles rows lo + R w .. + R, then + 8 R (R = kDfnInflight rows in flight).
// Rows move through buffer descriptors (one per row, lane offset 16 l,
// vector u at u * 1 KB): the range check zero-fills the vectors past the row
// and drops their stores.
#ifndef MDC_DFN_INFLIGHT
#define MDC_DFN_INFLIGHT 1
#endif
constexpr int kDfnInflight = MDC_DFN_INFLIGHT;
__device__ void dfn_copy_rows(const FfnDispatchIn& din, int8_t* __restrict__ q, float* __restrict__ scale, int lo,
                              int hi) {
  const int lane = threadIdx.x & 63;
  const int wv = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int nvec = din.nvec;
  for (int r = lo + kDfnInflight * wv; r < hi; r += kDfnInflight * (kFfnThreads / 64)) {
    v4u v[kDfnInflight][kQuantRowVec];
#pragma unroll
    for (int h = 0; h < kDfnInflight; ++h) {
      const int row = min(r + h, hi - 1);
      const int s = __builtin_amdgcn_readfirstlane(din.assist[(int64_t)row * 3]);
      const int t = __builtin_amdgcn_readfirstlane(din.assist[(int64_t)row * 3 + 1]);
      const __amdgpu_buffer_rsrc_t src = __builtin_amdgcn_make_buffer_rsrc(
          const_cast<v4u*>(din.x + ((int64_t)s * din.BS + t) * nvec), (short)0, nvec * 16, 0x00020000);
#pragma unroll
      for (int u = 0; u < kQuantRowVec; ++u)
        v[h][u] = __builtin_bit_cast(v4u, __builtin_amdgcn_raw_buffer_load_b128(src, (unsigned)lane * 16u,
                                                                                 (unsigned)u * 1024u, 0));
    }
#pragma unroll
    for (int h = 0; h < kDfnInflight; ++h) {
      const int row = r + h;
      if (row >= hi) break;
      uint64_t qv[kQuantRowVec];
      const float sc = quant_row<kQuantRowVec>(v[h], qv);
      const __amdgpu_buffer_rsrc_t dst =
          __builtin_amdgcn_make_buffer_rsrc(q + (int64_t)row * nvec * 8, (short)0, nvec * 8, 0x00020000);
#pragma unroll
      for (int u = 0; u < kQuantRowVec; ++u)
        __builtin_amdgcn_raw_buffer_store_b64(__builtin_bit_cast(v2u, qv[u]), dst, (unsigned)lane * 8u,
                                              (unsigned)u * 512u, 0);
      if (lane == 0) scale[row] = sc;
    }
  }
}

// Quantises the g rows [r0, r1) of one m-tile (the last GMM1 tile of the
// m-tile does it): codes clamp(rint(g * (127 / amax)), -127, 127) and scale
// amax / 127, with amax the row's max |g| gathered by the GMM1 epilogues,
// decided in fp32 as k_ffn_quant_rows decides them.  inv_s: kFfnBM floats of
// LDS.  One workgroup moves the whole m-tile, so it keeps 16 vectors per
// thread in flight.
__device__ void ffn_quant_mtile(const uint16_t* __restrict__ gsrc, int ncols, int8_t* __restrict__ q,
                                float* __restrict__ scale, const uint32_t* __restrict__ amax_bits, int r0, int r1,
                                float* inv_s) {
  const int tid = threadIdx.x;
  const int rows = r1 - r0;   // at most kFfnBM
  // the m-tile's row scales first, with 127 / amax kept in LDS (inv_s)
  if (tid < rows) {
    const float amax = __uint_as_float(amax_bits[r0 + tid]);
    inv_s[tid] = amax > 0.f ? 127.0f / amax : 0.f;
    scale[r0 + tid] = amax / 127.0f;
  }
  __syncthreads();
  const int nvec = ncols / 8;
  const int total = rows * nvec;
  constexpr int kBatch = 16;   // independent vectors in flight per thread
  for (int base = 0; base < total; base += kFfnThreads * kBatch) {
    v4u v[kBatch];
#pragma unroll
    for (int j = 0; j < kBatch; ++j) {
      const int idx = base + j * kFfnThreads + tid;
      const int row = r0 + idx / nvec;
      v[j] = idx < total ? *reinterpret_cast<const v4u*>(gsrc + (int64_t)row * ncols + (idx % nvec) * 8)
                         : v4u{0u, 0u, 0u, 0u};
    }
#pragma unroll
    for (int j = 0; j < kBatch; ++j) {
      const int idx = base + j * kFfnThreads + tid;
      if (idx >= total) continue;
      const int rr = idx / nvec;
      const float inv = inv_s[rr];
      uint64_t packed = 0;
#pragma unroll
      for (int w = 0; w < 4; ++w) {
        const float a = fminf(fmaxf(rintf(bf16_lo(v[j][w]) * inv), -127.f), 127.f);
        const float b = fminf(fmaxf(rintf(bf16_hi(v[j][w]) * inv), -127.f), 127.f);
        packed |= (uint64_t)(uint8_t)(int8_t)(int)a << (16 * w);
        packed |= (uint64_t)(uint8_t)(int8_t)(int)b << (16 * w + 8);
      }
      *reinterpret_cast<uint64_t*>(q + (int64_t)(r0 + rr) * ncols + (idx % nvec) * 8) = packed;
    }
  }
}

// The [PTO] fused pipeline as one persistent kernel: GMM1 + SwiGLU, the
// dynamic quantisation of g and GMM2 ([PTO] Overall Architecture: stages
// joined by ready flags), and with DISPATCH also the dispatch of the rows
// (mdc_dispatch_ffn).  Workgroups take items from one queue.
//
// Without DISPATCH the queue holds every GMM1 tile (plan order), then every
// GMM2 tile.  With DISPATCH it starts with the dispatch items of the first
// kDfnLead m-tiles (kDfnParts items of kFfnBM / kDfnParts rows per m-tile),
// then for j = 0 .. MT - 1 the dispatch items of m-tile j + kDfnLead
// followed by GMM1 tiles j*nn1 .. (j + 1)*nn1 - 1, then the GMM2 tiles: an
// m-tile's rows are dispatched while GMM1 runs on the m-tiles before it
// ([PTO] Dispatch of group i + 1 beside GMM1 of group i, D2C flags).  GMM1
// tile t belongs to a chunk of at most kFfnChunkM = kDfnLead m-tiles that
// starts at or before m-tile t / nn1, so every m-tile it reads had all of
// its dispatch items earlier in the queue.
//
// A dispatch item writes its rows' codes and scales and adds its row count
// to rows_ready[m]; a GMM1 tile waits until rows_ready[m] covers its m-tile.
// A GMM1 tile stores its g tile, folds max |g| per row into amax_bits and
// counts itself in done1[m]; the workgroup that finishes an m-tile's last
// GMM1 tile quantises the m-tile's g rows ([PTO] segmented SwiGLU: one
// segment per m-tile) and sets ready[m] (C2V / V2C flags); a GMM2 tile waits
// for ready[m].  Every wait is on an item that left the queue earlier, and
// items that left the queue are run by workgroups that are running, so every
// wait ends; each one is also bounded by spin_limit polls (one that runs out
// is counted in the status block's wait_timeouts and its tile written as
// NaN).  The XCDs' L2s are not coherent with each other: writes are
// published with agent-scope release fences (ffn_publish_begin: one L2
// write-back per item); the quantiser reads g after one acquire (an L2
// invalidate) per m-tile, and tiles read rows written in the same launch
// (dispatched q1 and s1, quantised q2 and s2) with agent-coherent loads
// instead of invalidating their XCD's L2 once per tile.
constexpr int kDfnParts = 8;               // dispatch items per m-tile
constexpr int kDfnRows = kFfnBM / kDfnParts;
constexpr int kDfnLead = kFfnChunkM;       // m-tiles dispatched ahead of GMM1
static_assert(kDfnLead >= kFfnChunkM, "a chunk's m-tiles must be dispatched before its first GMM1 tile");

template <bool TAB, bool DISPATCH>
__global__ __launch_bounds__(kFfnThreads) void k_ffn_fused(FfnGemm g1, FfnGemm g2, const int4* __restrict__ tiles,
                                                            FfnSync sync, int spin_limit, FfnDispatchIn din) {
  __shared__ __attribute__((aligned(16))) uint8_t lds0[kFfnStage];
  __shared__ __attribute__((aligned(16))) uint8_t lds1[kFfnStage];
  __shared__ float sc_row[kFfnBM];
  __shared__ float sc_col[kFfnBW];
  __shared__ int4 tab_s[TAB ? kFfnTabCache : 1];
  __shared__ int bcast[2];
  const FfnSmem sm{lds0, lds1, sc_row, sc_col, nullptr, nullptr};
  const int tid = threadIdx.x;
  const int MT = __builtin_amdgcn_readfirstlane(tiles[0].x);
  ffn_cache_tab<TAB>(tiles, tab_s, MT);
  const FfnTab<TAB> tab{tiles, tab_s};
  const int nn1 = (g1.Nout + kFfnBW / 2 - 1) / (kFfnBW / 2);
  const int nn2 = (g2.Nout + kFfnBW - 1) / kFfnBW;
  const int PRO = DISPATCH ? kDfnParts * min(kDfnLead, MT) : 0;
  const int T1 = DISPATCH ? PRO + MT * (kDfnParts + nn1) : MT * nn1;
  const int TT = T1 + MT * nn2;
  const auto no_next = []() { return FfnNext{false, int4{0, 0, 0, 0}, 0}; };
  for (;;) {
    __syncthreads();   // bcast is free
    if (tid == 0) bcast[0] = atomicAdd(sync.next, 1);
    __syncthreads();
    const int t = __builtin_amdgcn_readfirstlane(bcast[0]);
    if (t >= TT) break;
    FfnStage0 s0;
    if (t < T1) {
      int t1 = t;
      if (DISPATCH) {
        int item = t;   // dispatch item (m-tile * kDfnParts + part), or -1
        if (t >= PRO) {
          const int j = (t - PRO) / (kDfnParts + nn1), r = t - PRO - j * (kDfnParts + nn1);
          item = r < kDfnParts ? (j + kDfnLead) * kDfnParts + r : -1;
          t1 = j * nn1 + (r - kDfnParts);
        }
        if (item >= 0) {
          const int m = item / kDfnParts;
          if (m >= MT) continue;   // past the last m-tile: nothing to dispatch
          const int4 ti = tab.at(m);
          const int lo = ti.y + (item - m * kDfnParts) * kDfnRows;
          const int hi = min(min(ti.z, ti.y + kFfnBM), lo + kDfnRows);
          if (lo >= hi) continue;
          dfn_copy_rows(din, const_cast<int8_t*>(g1.a_src), const_cast<float*>(g1.row_scale), lo, hi);
          ffn_publish_begin();
          if (tid == 0) atomicAdd(sync.rows_ready + m, hi - lo);
          continue;
        }
      }
      int mt, nt;
      ffn_decode_tile(t1, nn1, tab, mt, nt);
      const int4 ti = tab.at(mt);
      bool late = false;
      if (DISPATCH) {
        if (tid == 0)
          bcast[1] = ffn_wait_at_least(sync.rows_ready + mt, min(ti.z, ti.y + kFfnBM) - ti.y, spin_limit,
                                       sync.status);
        __syncthreads();
        late = bcast[1] != 0;
      }
      if (late) {
        ffn_poison_tile(g1, ti, nt, kFfnBW / 2, sync.amax_bits);
      } else {
        // dispatched rows are read with agent-coherent loads
        ffn_tile<true, DISPATCH, false, false>(g1, ti, nt, sm, sync.amax_bits, s0, false, s0, no_next);
      }
      // Publish the g tile (and max |g|) before counting it.
      ffn_publish_begin();
      if (tid == 0) {
        const bool last = atomicAdd(sync.done1 + mt, 1) == nn1 - 1;
        if (last) __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "agent");   // see the other tiles' g and amax
        bcast[1] = last;
      }
      __syncthreads();
      if (bcast[1]) {
        ffn_quant_mtile(g1.out, g1.Nout, const_cast<int8_t*>(g2.a_src), const_cast<float*>(g2.row_scale),
                        sync.amax_bits, ti.y, min(ti.z, ti.y + kFfnBM), sm.sc_row);
        __syncthreads();
        // release q2 and s2 with the flag
        if (tid == 0) __hip_atomic_store(sync.ready + mt, 1, __ATOMIC_RELEASE, __HIP_MEMORY_SCOPE_AGENT);
      }
    } else {
      int mt, nt;
      ffn_decode_tile(t - T1, nn2, tab, mt, nt);
      if (tid == 0) bcast[1] = ffn_wait_at_least(sync.ready + mt, 1, spin_limit, sync.status);
      __syncthreads();
      if (bcast[1]) {
        ffn_poison_tile(g2, tab.at(mt), nt, kFfnBW, nullptr);
        continue;
      }
      // q2 and s2 are read with agent-coherent loads (no L2 invalidate)
      ffn_tile<false, true, false, false>(g2, tab.at(mt), nt, sm, nullptr, s0, false, s0, no_next);
    }
  }
}

// ---------------------------------------------------------------------------
// Host side
// ---------------------------------------------------------------------------
struct FfnPlan {
  int64_t A;
  int H, N, L;
  size_t off_q1, off_s1, off_g, off_q2, off_s2, off_tiles, off_amax, off_sync, bytes;
};

// Workspace: [status block][q1][s1][g][q2][s2][m-tile table][amax][sync words].
FfnPlan make_ffn_plan(const mdc_shape* sh, int inter_n) {
  FfnPlan f;
  f.A = sh->capacity;
  f.H = sh->hidden;
  f.N = inter_n;
  f.L = sh->num_experts / sh->world;
  f.off_q1 = MDC_STATUS_BYTES;
  f.off_s1 = f.off_q1 + round_up((size_t)f.A * f.H, 256);
  f.off_g = f.off_s1 + round_up((size_t)f.A * 4, 256);
  f.off_q2 = f.off_g + round_up((size_t)f.A * (f.N / 2) * 2, 256);
  f.off_s2 = f.off_q2 + round_up((size_t)f.A * (f.N / 2), 256);
  f.off_tiles = f.off_s2 + round_up((size_t)f.A * 4, 256);
  // m-tile table: header + at most A / kFfnBM + L tiles
  const size_t max_mtiles = 2 + f.A / kFfnBM + f.L;
  f.off_amax = f.off_tiles + round_up(max_mtiles * sizeof(int4), 256);
  f.off_sync = f.off_amax + round_up((size_t)f.A * 4, 256);
  f.bytes = f.off_sync + round_up(FfnSyncLayout::words((int)max_mtiles, f.L) * sizeof(int), 256);
  return f;
}

mdc_status check_ffn(const mdc_shape* sh, int inter_n) {
  const mdc_status st = check_shape(sh);
  if (st != MDC_OK) return st;
  if (inter_n <= 0) return MDC_ERR_INVALID;
  if ((inter_n % (2 * kFfnOutAlign)) != 0) return MDC_ERR_UNSUPPORTED;
  if ((sh->hidden % kFfnOutAlign) != 0) return MDC_ERR_UNSUPPORTED;
  // one expert's weight matrix (N x H or H x N/2 bytes) is addressed with 32-bit offsets
  if ((int64_t)inter_n * sh->hidden > INT32_MAX) return MDC_ERR_UNSUPPORTED;
  // tiles of both GEMMs (and the work-queue tickets) are counted in 32 bits
  const int64_t L = sh->num_experts / sh->world;
  const int64_t max_mtiles = 2 + sh->capacity / kFfnBM + L;
  const int64_t per_mtile = inter_n / kFfnBW + (sh->hidden + kFfnBW - 1) / kFfnBW;
  if (max_mtiles * per_mtile + 65536 > INT32_MAX) return MDC_ERR_UNSUPPORTED;
  return MDC_OK;
}

// GMM1 -> quantise g -> GMM2 runs as three stream-ordered kernels, or as
// the one persistent k_ffn_fused launch with MDC_FLAG_FFN_PIPELINE (the
// results are identical; the stream-ordered GEMMs load each next tile ahead
// and measure faster).  Polls of a GMM2 tile's wait before it gives up:
// 2^24, or 2^s with s from the flags' spin field.
int ffn_spin_limit(uint32_t flags) {
  const uint32_t sft = (flags & MDC_FLAG_SPIN_MASK) >> MDC_FLAG_SPIN_SHIFT;
  return sft != 0 ? (1 << (sft > 30 ? 30 : sft)) : (1 << 24);
}

// Capacity of the m-tile table, and the fused kernel's synchronisation
// words (w = NULL for the stream-ordered kernels, which use none).
int ffn_max_mtiles(const FfnPlan& f) { return (int)(2 + f.A / kFfnBM + f.L); }

FfnSyncLayout ffn_sync_layout(const FfnPlan& f, char* ws, bool fused) {
  return FfnSyncLayout{fused ? reinterpret_cast<int*>(ws + f.off_sync) : nullptr, ffn_max_mtiles(f), f.L};
}

FfnSync ffn_sync(const FfnSyncLayout& sw, uint32_t* amax, mdc_device_status* status) {
  return FfnSync{sw.next(), sw.done1(), sw.ready(), sw.rows_ready(), amax, status};
}

// Workgroups of the persistent GEMM launches: one per CU (128 KB of LDS
// each), a multiple of 8 so that every XCD gets the same number.
unsigned ffn_persistent_grid() {
  int dev = 0, cus = 256;
  if (hipGetDevice(&dev) == hipSuccess) (void)hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev);
  return (unsigned)(((cus + 7) / 8) * 8);
}

mdc_status ffn_impl(const FfnPlan& f, uint32_t flags, const void* expand_x, const int8_t* expand_q,
                    const float* dyn_scale, const int64_t* expert_token_nums, const int8_t* w1, const float* w1_scale,
                    const int8_t* w2, const float* w2_scale, void* y, char* ws, hipStream_t s) {
  mdc_device_status* status = reinterpret_cast<mdc_device_status*>(ws);
  int8_t* q1 = reinterpret_cast<int8_t*>(ws + f.off_q1);
  float* s1 = reinterpret_cast<float*>(ws + f.off_s1);

  uint16_t* g = reinterpret_cast<uint16_t*>(ws + f.off_g);
  int8_t* q2 = reinterpret_cast<int8_t*>(ws + f.off_q2);
  float* s2 = reinterpret_cast<float*>(ws + f.off_s2);
  const unsigned g1 = ffn_persistent_grid(), g2 = g1;
  const unsigned quant_wgs = g1 * 8;
  (void)hipGetLastError();
  if (expand_q == nullptr) {
    launch_quant_rows(static_cast<const v4u*>(expand_x), q1, s1, expert_token_nums, f.L, f.A, f.H / 8, quant_wgs, s);
  } else {
    q1 = const_cast<int8_t*>(expand_q);   // rows already quantised by mdc_dispatch_quant
    s1 = const_cast<float*>(dyn_scale);
  }
  int4* tiles = reinterpret_cast<int4*>(ws + f.off_tiles);
  uint32_t* amax = reinterpret_cast<uint32_t*>(ws + f.off_amax);
  const FfnGemm gemm1{q1, s1, w1, w1_scale, g, f.H, f.N, f.N / 2};
  const FfnGemm gemm2{q2, s2, w2, w2_scale, static_cast<uint16_t*>(y), f.N / 2, f.H, f.H};
  const bool fused = (flags & MDC_FLAG_FFN_PIPELINE) != 0;
  const FfnSyncLayout sw = ffn_sync_layout(f, ws, fused);
  hipLaunchKernelGGL(k_ffn_plan, dim3(1), dim3(kPlanThreads), 0, s, expert_token_nums, f.L, f.A, tiles, sw, amax,
                     status);
  if (fused) {
    const bool tab = sw.stride <= kFfnTabCache;   // the m-tile table fits in LDS
    const FfnSync sync = ffn_sync(sw, amax, status);
    const int spin = ffn_spin_limit(flags);
    const FfnDispatchIn none{nullptr, nullptr, 0, 0};
    if (tab)
      hipLaunchKernelGGL((k_ffn_fused<true, false>), dim3(g1), dim3(kFfnThreads), 0, s, gemm1, gemm2, tiles, sync,
                         spin, none);
    else
      hipLaunchKernelGGL((k_ffn_fused<false, false>), dim3(g1), dim3(kFfnThreads), 0, s, gemm1, gemm2, tiles, sync,
                         spin, none);
  } else {
    const bool tab = sw.stride <= kFfnTabCacheExt;
    if (tab)
      hipLaunchKernelGGL((k_ffn_gemm<true, true>), dim3(g1), dim3(kFfnThreads), 0, s, gemm1, tiles);
    else
      hipLaunchKernelGGL((k_ffn_gemm<true, false>), dim3(g1), dim3(kFfnThreads), 0, s, gemm1, tiles);
    launch_quant_rows(reinterpret_cast<const v4u*>(g), q2, s2, expert_token_nums, f.L, f.A, f.N / 2 / 8, quant_wgs, s);
    if (tab)
      hipLaunchKernelGGL((k_ffn_gemm<false, true>), dim3(g2), dim3(kFfnThreads), 0, s, gemm2, tiles);
    else
      hipLaunchKernelGGL((k_ffn_gemm<false, false>), dim3(g2), dim3(kFfnThreads), 0, s, gemm2, tiles);
  }
  return launched();
}

// mdc_dispatch_ffn: the plan (scan of the layout's group counters + FFN
// tile plan), the route placement, then the persistent pipeline with the
// dispatch items in its queue.
mdc_status dispatch_ffn_impl(const DispatchPlan& p, const FfnPlan& f, uint32_t flags, const void* x,
                             const GatherMeta& m, int8_t* expand_q, float* dyn_scale, const int8_t* w1,
                             const float* w1_scale, const int8_t* w2, const float* w2_scale, void* y, char* dws,
                             char* fws, hipStream_t s) {
  int32_t* base = reinterpret_cast<int32_t*>(dws + p.off_base);
  int4* tiles = reinterpret_cast<int4*>(fws + f.off_tiles);
  uint32_t* amax = reinterpret_cast<uint32_t*>(fws + f.off_amax);
  mdc_device_status* fstatus = reinterpret_cast<mdc_device_status*>(fws);
  const FfnSyncLayout sw = ffn_sync_layout(f, fws, true);
  (void)hipGetLastError();
  hipLaunchKernelGGL(k_dfn_plan, dim3(1), dim3(kPlanThreads), 0, s, m.cnt, m.drop, base, p.L, p.W, p.G, p.A,
                     m.ep_recv, m.expert_nums, m.status, tiles, sw, amax, fstatus);
  const int n_routes = p.W * p.BS * p.K;
  if (n_routes > 0)
    hipLaunchKernelGGL(k_dfn_route, dim3((n_routes + 255) / 256), dim3(256), 0, s, m, base, p.BS, p.K, p.L, p.W,
                       p.TPG, p.G, p.A, n_routes);
  if (n_routes > 0 && f.A > 0) {
    const FfnGemm gemm1{expand_q, dyn_scale, w1, w1_scale, reinterpret_cast<uint16_t*>(fws + f.off_g), f.H, f.N,
                        f.N / 2};
    const FfnGemm gemm2{reinterpret_cast<int8_t*>(fws + f.off_q2), reinterpret_cast<float*>(fws + f.off_s2), w2,
                        w2_scale, static_cast<uint16_t*>(y), f.N / 2, f.H, f.H};
    const FfnSync sync = ffn_sync(sw, amax, fstatus);
    const FfnDispatchIn din{static_cast<const v4u*>(x), m.assist, p.BS, p.nvec};
    const int spin = ffn_spin_limit(flags);
    const unsigned grid = ffn_persistent_grid();
    if (sw.stride <= kFfnTabCache)
      hipLaunchKernelGGL((k_ffn_fused<true, true>), dim3(grid), dim3(kFfnThreads), 0, s, gemm1, gemm2, tiles, sync,
                         spin, din);
    else
      hipLaunchKernelGGL((k_ffn_fused<false, true>), dim3(grid), dim3(kFfnThreads), 0, s, gemm1, gemm2, tiles, sync,
                         spin, din);
  }
  return launched();
}

}  // namespace

extern "C" {

mdc_status mdc_ffn_workspace(const mdc_shape* shape, int32_t inter_n, size_t* bytes) {
  if (bytes == nullptr) return MDC_ERR_NULLPTR;
  const mdc_status st = check_ffn(shape, inter_n);
  if (st != MDC_OK) return st;
  *bytes = make_ffn_plan(shape, inter_n).bytes;
  return MDC_OK;
}

mdc_status mdc_ffn_workspace_size(const mdc_shape* shape, int32_t inter_n, size_t* bytes) {
  return mdc_ffn_workspace(shape, inter_n, bytes);
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
  return ffn_impl(f, (uint32_t)shape->flags, expand_x, nullptr, nullptr, expert_token_nums, w1, w1_scale, w2,
                  w2_scale, y, static_cast<char*>(workspace), static_cast<hipStream_t>(stream));
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
  return ffn_impl(f, (uint32_t)shape->flags, nullptr, expand_q, dynamic_scales, expert_token_nums, w1, w1_scale,
                  w2, w2_scale, y, static_cast<char*>(workspace), static_cast<hipStream_t>(stream));
}


mdc_status mdc_dispatch_ffn(const mdc_shape* shape, int32_t inter_n, const void* x, const float* expert_scales,
                            int8_t* expand_q, float* dynamic_scales, int32_t* assist_info, int32_t* ep_recv_counts,
                            int64_t* expert_token_nums, int32_t* expanded_row_idx, float* expand_scales,
                            const int8_t* w1, const float* w1_scale, const int8_t* w2, const float* w2_scale, void* y,
                            void* dispatch_workspace, size_t dispatch_workspace_bytes, void* ffn_workspace,
                            size_t ffn_workspace_bytes, void* stream) {
  mdc_status st = check_ffn(shape, inter_n);
  if (st != MDC_OK) return st;
  const DispatchPlan p = make_plan(shape);
  st = check_plan(p);
  if (st != MDC_OK) return st;
  st = check_gather_args(p, x, expand_q, dynamic_scales, true, assist_info, ep_recv_counts, expert_token_nums,
                         expanded_row_idx, expert_scales, expand_scales, dispatch_workspace, dispatch_workspace_bytes);
  if (st != MDC_OK) return st;
  const FfnPlan f = make_ffn_plan(shape, inter_n);
  if (ffn_workspace == nullptr) return MDC_ERR_NULLPTR;
  if (p.BS > 0 && f.A > 0 &&
      (w1 == nullptr || w1_scale == nullptr || w2 == nullptr || w2_scale == nullptr || y == nullptr))
    return MDC_ERR_NULLPTR;
  if (!aligned16(w1) || !aligned16(w2) || !aligned16(y)) return MDC_ERR_INVALID;
  if (ffn_workspace_bytes < f.bytes) return MDC_ERR_WORKSPACE;
  char* dws = static_cast<char*>(dispatch_workspace);
  const GatherMeta m = make_meta(p, dws, expert_scales, expand_scales, assist_info, ep_recv_counts,
                                 expert_token_nums, expanded_row_idx);
  return dispatch_ffn_impl(p, f, (uint32_t)shape->flags, x, m, expand_q, dynamic_scales, w1, w1_scale, w2, w2_scale,
                           y, dws, static_cast<char*>(ffn_workspace), static_cast<hipStream_t>(stream));
}

}  // extern "C"
