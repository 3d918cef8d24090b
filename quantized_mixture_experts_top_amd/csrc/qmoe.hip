// Fused int4 group-32 Mixture-of-Experts layer for AMD Instinct MI355X
// (gfx950): HIP kernels and the host side of the C ABI declared in qmoe.h.
//
// Steps of one call, all on the caller's stream:
//   route_single_kernel (calls of at most 64 tokens), or route_topk_kernel
//                   then route_finish_kernel: top-k routing, expert counts,
//                   their exclusive scan, the stable sort of routed slots by
//                   expert, the flat list of (expert, row tile) work items,
//                   x -> fp16 operand format
//   gemm_kernel<..., true>   stacked gate+up product with h = SiLU(g)*u
//   gemm_kernel<..., false>  down product times the routing weight
//                   (128-row MFMA tiles; calls averaging at most 1.75 routed
//                   rows per expert run gemv_kernel<..., true / false, NT>,
//                   the same two products as packed fp16 dot products)
//   combine_kernel  out[t] = sum over slots in order (+ shared expert)
//
// Layer definition: "The MoE Throughput Lever: Quantifying the INT4 Marlin
// GEMM on Blackwell PRO 6000" (sections "The Context: Why This Measurement
// Matters", "The Benchmark: What Was Measured"); per-expert counts and their
// scan: "Detailed results" (section "Nsight Compute on the stock kernel");
// sorted routing and the stacked gate+up GEMM: "perf(exl3): accelerate
// fat-expert prefill" (description, section "Rollout").
#include <hip/hip_runtime.h>

#include <algorithm>
#include <atomic>
#include <cstdio>
#include <mutex>
#include <cstdlib>
#include <cstring>
#include <string>
#include <type_traits>
#include <utility>
#include <vector>

#include "qmoe.h"
#include "qmoe_device.h"

using namespace qmoe;

namespace {

constexpr int kThreads = 256;   // every kernel: 4 waves of 64
constexpr int kChunk = 64;      // tokens per routing chunk = bits of one mask word
constexpr int kCtrlWords = 64;  // [1] work items, [2] a mixed call's dot-product items
constexpr int kKStep = 128;     // inputs per K-step of a wave (4 lane groups x 32)

// Shape of the 128-row MFMA tiles: MB row blocks of 16 per work item, NBW
// 16-column output blocks per wave (gate+up: each with its up block).
// 128-row tile shapes, measured on MI355X over 256..4096 tokens of the
// 384-expert 7168/2048 layer.  Gate+up: blocks of 4 waves, each two 16-column
// blocks of gate and their up blocks (64 weight rows per wave, so each
// activation fragment read from LDS feeds 4 MFMAs).  Down: blocks of 8
// waves, each one 16-column block; at under 128 registers four waves share
// a SIMD, which hides the activation-tile latency better than wider waves.
constexpr int kTileMB = 8;  // row blocks of 16 per tile
constexpr int kGuWN = 4, kGuNBW = 2, kGuWPE = 2;
constexpr int kDnWN = 8, kDnNBW = 1, kDnWPE = 4;
// Gate+up K loops of up to this many 16-row blocks issue their weights two
// sub-steps at a time: 2-4% faster at 90-1024 tokens on the 384-expert layer
// (measured with the codes in row order, where the two sub-steps were the
// halves of each row's 128-byte line).  Loops of 5-7 blocks fit the extra
// live fragment too (the 8-block loop spills it), but there pairing measured
// no faster at 90-1024 tokens and 1-2% slower at 4096 than the interleaved
// issue; in the down tiles pairing measured neutral to 3-5% slower.
constexpr int kGuPairRowBlocks = 4;
constexpr int kPrefillRows = kTileMB * 16;

// ---------------------------------------------------------------- routing

struct RouteArgs {
  const float* logits;
  const uint4* x;  // bf16 [M, H] as 16-byte runs
  int M, E, H, k, S, C, bmc, max_items;
  int nrb;  // blocks before the x-conversion blocks
  int* ctrl;
  int* ids;
  float* wts;
  int* counts;
  int* offsets;
  int* perm;
  int* inv_perm;
  int4* items;
  int4* items_gv;  // a mixed call: one dot-product item per expert of 1..gv rows (gv = 0: none)
  int gv;
  uint4* xa;   // fp16 A-format [M, H], row t times 2^-xexp[t]
  int* xexp;   // [M] per-token exponent
  int* tickets;    // the GEMV split-K tickets, cleared here for the call
  int n_tickets;
  int lo, nloc;    // local experts [lo, lo + nloc) (an expert-parallel shard; else 0, E)
  int scoring;            // QMOE_SCORING_SOFTMAX or QMOE_SCORING_SIGMOID
  float rscale;           // sigmoid: routed scaling factor
  const float* bias;      // sigmoid: per-expert selection bias [E] or nullptr
};

constexpr int kRouteThreads = 1024;  // routing blocks: up to 16 waves
constexpr int kRouteWaves = kRouteThreads / 64;  // also token rows per conversion block

// Counts, offsets and the flat work list from the per-expert row counts in
// s_cnt[0..E) (the caller's threads wrote them before calling), all in LDS.
// One wave does both exclusive scans (row offsets and work-item offsets)
// over the E+1 entries at once: lane l reads its run of ceil((E+1)/64)
// consecutive counts into registers, sums them, DPP scans combine the 64
// lane totals, and each lane walks its run again to write offsets and, when
// `write` is set, the counts, offsets and items to the workspace.  This
// replaces a serial loop over the expert counts, and needs no block barrier
// between the two scans.  The shared expert (entry E, a row per token) gets
// the first items: its tiles are the longest of a call and should not be
// the last to start.  Items hold a power of two rows (bmc), so the item
// counts are shifts.
constexpr int kMaxRun = (QMOE_MAX_EXPERTS + 1 + 63) / 64;  // counts per lane
__device__ void route_items(const RouteArgs& a, int* s_cnt, int* s_off, bool write) {
  const int tid = threadIdx.x, E = a.nloc, n = E + 1, bmc = a.bmc;  // over the local experts
  const int lg = 31 - __builtin_clz(bmc);
  if (tid == 0) s_cnt[E] = a.S;  // the shared expert takes every token
  __syncthreads();
  if (tid < 64) {
    const int lane = tid, per = (n + 63) / 64, e0 = lane * per;
    int cnt[kMaxRun];
#pragma unroll
    for (int u = 0; u < kMaxRun; ++u) cnt[u] = (u < per && e0 + u < n) ? s_cnt[e0 + u] : 0;
    // (a mixed call: a routed expert of 1..gv rows takes one dot-product
    // item instead of tile items)
    auto light = [&](int e, int c) { return e < E && c >= 1 && c <= a.gv; };
    int c_loc = 0, i_loc = 0, g_loc = 0;
#pragma unroll
    for (int u = 0; u < kMaxRun; ++u) {
      const bool lt = light(e0 + u, cnt[u]);
      c_loc += cnt[u];
      i_loc += lt ? 0 : (cnt[u] + bmc - 1) >> lg;
      g_loc += lt ? 1 : 0;
    }
    const int c_inc = wave_incl_scan_add(c_loc), i_inc = wave_incl_scan_add(i_loc);
    const int g_inc = a.gv ? wave_incl_scan_add(g_loc) : 0;
    const int nsh = (a.S + bmc - 1) >> lg;  // the shared expert's items
    int c_run = c_inc - c_loc, i_run = i_inc - i_loc, g_run = g_inc - g_loc;
#pragma unroll
    for (int u = 0; u < kMaxRun; ++u) {
      const int e = e0 + u;
      if (u >= per || e >= n) break;
      const int c = cnt[u];
      const bool lt = light(e, c);
      const int ni = lt ? 0 : (c + bmc - 1) >> lg;
      s_off[e] = c_run;
      if (write) {
        a.counts[e] = c;
        a.offsets[e] = c_run;
        const int base = e == E ? 0 : i_run + nsh;
        for (int i = 0; i < ni; ++i) {
          const int r0 = i << lg;
          if (base + i < a.max_items) a.items[base + i] = make_int4(e, r0, min(bmc, c - r0), c_run + r0);
        }
        if (lt) a.items_gv[g_run] = make_int4(e, 0, c, c_run);
      }
      c_run += c;
      i_run += ni;
      g_run += lt ? 1 : 0;
    }
    if (lane == 63) {
      s_off[n] = c_run;
      if (write) {
        a.offsets[n] = c_run;
        a.ctrl[1] = min(i_run, a.max_items);
        a.ctrl[2] = g_run;
      }
    }
  }
  __syncthreads();
}

// Sigmoid score s = 1 / (1 + e^-l) in fp32, formed as q = min(s, 1 - s) from
// e^-|l| <= 1 and then s = 1 - q for l >= 0: one rounding near 1 (rounding
// 1 + e^-l first would reach 1.0 a factor of two early in e^-l), and no
// overflow of e^-l for l << 0.
__device__ __forceinline__ float sigmoid_score(float l) {
  const float e = expf(-fabsf(l));
  const float q = e / (1.0f + e);
  return l >= 0.0f ? 1.0f - q : q;
}

// The top_k experts of token t (one wave): order-preserving keys held in
// registers; each of k rounds takes the largest key and, among experts
// holding it, the lowest index.  Lane j < k returns the j-th selection and
// its weight.  EPL = logits per lane (E <= 64 * EPL).  The key is the logit
// (softmax scoring) or, for the sigmoid scoring, the fp32 score
// s = 1 / (1 + e^-l) plus the expert's selection bias.
// (in two parts: the row's loads, issued early where the caller has other
// work to overlap with their trip to memory, and the selection)
template <int EPL>
struct TopkRow {
  float lv[EPL], bv[EPL];
};
template <int EPL>
__device__ __forceinline__ void topk_load(const RouteArgs& a, int t, int lane, TopkRow<EPL>& r) {
  const int E = a.E;
  const float* row = a.logits + (size_t)t * E;
  // (loads clamped into the row rather than predicated, so they all issue
  // before the first wait)
#pragma unroll
  for (int s = 0; s < EPL; ++s) r.lv[s] = row[min(s * 64 + lane, E - 1)];
  if (a.scoring == QMOE_SCORING_SIGMOID) {
#pragma unroll
    for (int s = 0; s < EPL; ++s) r.bv[s] = a.bias ? a.bias[min(s * 64 + lane, E - 1)] : 0.0f;
  }
}
template <int EPL>
__device__ __forceinline__ void topk_pick(const RouteArgs& a, int t, int lane, const TopkRow<EPL>& r, int& my_e,
                                          float& my_w) {
  const int E = a.E, k = a.k;
  const bool sig = a.scoring == QMOE_SCORING_SIGMOID;
  const float* row = a.logits + (size_t)t * E;
  const float* lv = r.lv;
  const float* bv = r.bv;
  // (absent and taken experts have key 0, below every finite value's)
  uint32_t key[EPL];
#pragma unroll
  for (int s = 0; s < EPL; ++s) key[s] = (s * 64 + lane < E) ? ordered_key(sig ? sigmoid_score(lv[s]) + bv[s] : lv[s]) : 0u;
  my_e = 0;
  float my_l = 0.0f;
  for (int j = 0; j < k; ++j) {
    uint32_t best = 0;
#pragma unroll
    for (int s = 0; s < EPL; ++s) best = key[s] > best ? key[s] : best;
    best = wave_max_u32(best);
    int e_sel = -1;
#pragma unroll
    for (int s = 0; s < EPL; ++s) {
      const uint64_t m = __ballot(key[s] == best);
      if (e_sel < 0 && m != 0) e_sel = s * 64 + __ffsll((long long)m) - 1;
    }
#pragma unroll
    for (int s = 0; s < EPL; ++s)
      if (s * 64 + lane == e_sel) key[s] = 0;
    if (lane == j) {
      my_e = e_sel;
      my_l = from_ordered_key(best);
    }
  }
  if (sig) {
    // the selected scores (the same arithmetic again, from the logit: a read
    // of the row just loaded) renormalised, times the routed scaling factor
    const float my_s = lane < k ? sigmoid_score(row[my_e]) : 0.0f;
    float sum = my_s;
#pragma unroll
    for (int m = 32; m >= 1; m >>= 1) sum += __shfl_xor(sum, m, 64);
    my_w = my_s / sum * a.rscale;
    return;
  }
  // renormalised softmax over the selected logits: the full-softmax
  // denominator cancels, so w_j = exp(l_j - l_0) / sum_j' exp(l_j' - l_0)
  const float lj = (lane < k) ? my_l : 0.0f;
  const float l0 = __shfl(lj, 0, 64);
  const float ex = (lane < k) ? expf(lj - l0) : 0.0f;
  float sum = ex;
#pragma unroll
  for (int m = 32; m >= 1; m >>= 1) sum += __shfl_xor(sum, m, 64);
  my_w = ex / sum;
}
template <int EPL>
__device__ __forceinline__ void wave_topk(const RouteArgs& a, int t, int lane, int& my_e, float& my_w) {
  TopkRow<EPL> r;
  topk_load<EPL>(a, t, lane, r);
  topk_pick<EPL>(a, t, lane, r, my_e, my_w);
}

// x -> fp16 operand format, one wave per token row: the row's largest |x|
// sets its exponent e, and the row is stored times 2^-e (exact), so any
// finite bf16 row fits fp16.  A lane holds up to kConvRuns runs of 8 inputs
// (rows of up to 8192 inputs whole), all requested before the first is
// used, so a row costs one trip to memory and is converted from registers;
// a longer row goes in chunks of that size and is read a second time.
constexpr int kConvRuns = 16;
__device__ __forceinline__ void convert_x_row(const RouteArgs& a, int t, int lane) {
  const int runs = a.H / 8;
  const uint4* __restrict__ row = a.x + (size_t)t * runs;
  uint4* __restrict__ dst = a.xa + (size_t)t * runs;
  uint4 r[kConvRuns];
  uint32_t amax = 0;
  for (int c0 = 0; c0 < runs; c0 += 64 * kConvRuns) {
#pragma unroll
    for (int u = 0; u < kConvRuns; ++u) {
      const int v = c0 + u * 64 + lane;
      r[u] = v < runs ? row[v] : make_uint4(0u, 0u, 0u, 0u);
    }
#pragma unroll
    for (int u = 0; u < kConvRuns; ++u) amax = max(amax, absmax_bf16x8(r[u]));
  }
  const int e = row_exponent(wave_max_u32(amax));
  const float sc = pow2f(-e);
  if (lane == 0) a.xexp[t] = e;
  if (runs <= 64 * kConvRuns) {  // the row is still in r
#pragma unroll
    for (int u = 0; u < kConvRuns; ++u) {
      const int v = u * 64 + lane;
      if (v < runs) dst[v] = bf16x8_to_aformat(r[u], sc);
    }
    return;
  }
  for (int v = lane; v < runs; v += 64) dst[v] = bf16x8_to_aformat(row[v], sc);  // long rows: again, from cache
}

// A call of at most 64 tokens is routed by one block of one wave per token
// (blockDim.x = 64 * min(M, 16)), which finishes in LDS: per-expert 64-bit
// masks of the tokens that chose it give each routed slot's rank inside its
// expert (popcount of the lower bits).  The blocks after it convert x.
template <int EPL>
__global__ __launch_bounds__(kRouteThreads) void route_single_kernel(RouteArgs a) {
  __shared__ uint32_t cm[QMOE_MAX_EXPERTS][2];
  __shared__ int s_cnt[QMOE_MAX_EXPERTS + 2];
  __shared__ int s_off[QMOE_MAX_EXPERTS + 2];
  __shared__ int s_ids[kChunk * QMOE_MAX_TOPK];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6, nthr = blockDim.x, nw = nthr / 64;
  const int E = a.E, k = a.k;
  if (blockIdx.x >= 1) {
    const int t = ((int)blockIdx.x - 1) * nw + wave;
    if (t < a.M) convert_x_row(a, t, lane);
    return;
  }
  // each wave's first token row goes out before the clears, which then
  // overlap its trip to memory (up to 512 experts: with more, the row does
  // not fit the registers left across the clears)
  constexpr bool kEarly = EPL <= 8;
  TopkRow<EPL> row;
  if (kEarly && wave < a.M) topk_load<EPL>(a, wave, lane, row);
  for (int e = tid; e < E; e += nthr) cm[e][0] = cm[e][1] = 0u;
  for (int i = tid; i < a.n_tickets; i += nthr) a.tickets[i] = 0;
  __syncthreads();
  for (int t = wave; t < a.M; t += nw) {
    int my_e;
    float my_w;
    if (!kEarly || t != wave) topk_load<EPL>(a, t, lane, row);
    topk_pick<EPL>(a, t, lane, row, my_e, my_w);
    if (lane < k) {
      a.ids[(size_t)t * k + lane] = my_e;
      a.wts[(size_t)t * k + lane] = my_w;
      s_ids[t * k + lane] = my_e;
      atomicOr(&cm[my_e][t >> 5], 1u << (t & 31));
    }
  }
  __syncthreads();
  for (int le = tid; le < a.nloc; le += nthr) s_cnt[le] = __popc(cm[a.lo + le][0]) + __popc(cm[a.lo + le][1]);
  route_items(a, s_cnt, s_off, true);
  // slot (t, j): its expert's offset plus the number of lower tokens routed
  // to that expert (each token selects an expert at most once); slots of
  // experts that are not local get no position
  for (int f = tid; f < a.M * k; f += nthr) {
    const int t = f / k, e = s_ids[f], le = e - a.lo;
    if (le < 0 || le >= a.nloc) {
      a.inv_perm[f] = -1;
      continue;
    }
    const unsigned long long m = (unsigned long long)cm[e][0] | ((unsigned long long)cm[e][1] << 32);
    const int pos = s_off[le] + __popcll(m & ((1ull << t) - 1ull));
    a.perm[pos] = f;
    a.inv_perm[f] = pos;
  }
  // the shared expert's rows follow the routed ones: slot T + t
  const int T = a.M * k;
  for (int t = tid; t < a.S; t += nthr) a.perm[s_off[a.nloc] + t] = T + t;
}

// Calls of more than 64 tokens, first of two kernels: one wave per token
// selects its top_k experts and weights (blocks of 16 tokens, spread over
// the GPU); the blocks after the routing blocks convert x.
template <int EPL>
__global__ __launch_bounds__(kRouteThreads) void route_topk_kernel(RouteArgs a) {
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  if ((int)blockIdx.x >= a.nrb) {
    const int t = ((int)blockIdx.x - a.nrb) * kRouteWaves + wave;
    if (t < a.M) convert_x_row(a, t, lane);
    return;
  }
  const int t = (int)blockIdx.x * kRouteWaves + wave;
  if (t >= a.M) return;
  int my_e;
  float my_w;
  wave_topk<EPL>(a, t, lane, my_e, my_w);
  if (lane < a.k) {
    a.ids[(size_t)t * a.k + lane] = my_e;
    a.wts[(size_t)t * a.k + lane] = my_w;
  }
}

// Second kernel: one block per chunk of 64 tokens.  Every block histograms
// all routed slots (the expert counts) and, separately, those of the tokens
// before its chunk; the counts' exclusive scan (route_items) plus the
// earlier tokens' count gives the first sorted position of the chunk's
// tokens in each expert, and the chunk's own per-expert token masks give
// each slot's rank after them.  So no block waits for another, and no
// global atomics or cleared memory are needed.  Block 0 also writes the
// counts, offsets and work items.
__global__ __launch_bounds__(kRouteThreads) void route_finish_kernel(RouteArgs a) {
  __shared__ uint32_t cm[QMOE_MAX_EXPERTS][2];
  __shared__ int s_cnt[QMOE_MAX_EXPERTS + 2];
  __shared__ int s_off[QMOE_MAX_EXPERTS + 2];
  __shared__ int s_before[QMOE_MAX_EXPERTS];
  const int tid = threadIdx.x, E = a.E, k = a.k, c = blockIdx.x;
  const int t0 = c * kChunk, rows = min(kChunk, a.M - t0);
  for (int i = c * kRouteThreads + tid; i < a.n_tickets; i += (int)gridDim.x * kRouteThreads) a.tickets[i] = 0;
  const int lo = a.lo, nloc = a.nloc;  // local experts (indices below are local)
  for (int e = tid; e < nloc; e += kRouteThreads) {
    s_cnt[e] = 0;
    s_before[e] = 0;
    cm[e][0] = cm[e][1] = 0u;
  }
  __syncthreads();
  const int T = a.M * k, before = t0 * k;
  const int* __restrict__ ids = a.ids;
  for (int f0 = 0; f0 < T; f0 += 4 * kRouteThreads) {  // four loads in flight per thread
    int e[4];
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      const int f = f0 + u * kRouteThreads + tid;
      e[u] = f < T ? ids[f] : -1;
    }
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      const int f = f0 + u * kRouteThreads + tid;
      const int le = e[u] - lo;
      if (e[u] < 0 || e[u] >= E || le < 0 || le >= nloc) continue;  // not local (or out of range)
      atomicAdd(&s_cnt[le], 1);
      if (f < before) atomicAdd(&s_before[le], 1);
      else if (f < before + rows * k) {
        const int tl = f / k - t0;
        atomicOr(&cm[le][tl >> 5], 1u << (tl & 31));
      }
    }
  }
  __syncthreads();
  route_items(a, s_cnt, s_off, c == 0);
  for (int f = before + tid; f < before + rows * k; f += kRouteThreads) {
    const int tl = f / k - t0, le = ids[f] - lo;
    if (le < 0 || le >= nloc) {
      a.inv_perm[f] = -1;
      continue;
    }
    const unsigned long long m = (unsigned long long)cm[le][0] | ((unsigned long long)cm[le][1] << 32);
    const int pos = s_off[le] + s_before[le] + __popcll(m & ((1ull << tl) - 1ull));
    a.perm[pos] = f;
    a.inv_perm[f] = pos;
  }
  for (int t = t0 + tid; t < t0 + rows && t < a.S; t += kRouteThreads) a.perm[s_off[nloc] + t] = T + t;
}

// ------------------------------------------------------------------ GEMMs

struct GemmArgs {
  const uint8_t* w;    // routed experts' codes  [E, Nw, K/2]
  const uint16_t* s;   // routed experts' scales [E, Nw, K/32]
  const uint8_t* w_sh; // shared expert (may be null)
  const uint16_t* s_sh;
  int E, K, N, Nw, nblk, max_items, T, k, M, R;
  const int* ctrl;
  int count_at;  // the ctrl word holding the item count: 1, or 2 for a mixed call's dot-product items
  const int4* items;
  const int* perm;
  const float* wts;
  const int* xexp;    // [M] per-token exponent e: x rows are held times 2^-e, h rows times 2^-2e
  const _Float16* a;  // A rows in A-format: x (gate+up) or h (down)
  uint32_t a_bytes;      // bytes of the A buffer (loads past it read 0)
  _Float16* h_out;    // gate+up: h [R, N] in A-format
  uint16_t* y_out;    // down: y [R, N] bf16 in slot order
  // GEMV split-K: K split over `splits` blocks per (item, column block);
  // fp32 partials [tiles][splits][256] and one ticket per tile (zeroed by
  // the routing kernels; the last arriver sets its ticket back to zero)
  int splits;
  float* part;
  int* tickets;
};

template <int NBB>
struct Frag {
  u32x4_t b[NBB];  // 32 packed codes of this lane's weight row per block
};

__device__ __forceinline__ uint32_t word(const u32x4_t& v, int i) { return v[i]; }

// Lane swaps between the 16-lane rows of a wave: (rows of a, rows of b)
// become (a0 b0 a2 b2, a1 b1 a3 b3) for 16 and (a0 a1 b0 b1, a2 a3 b2 b3)
// for 32.
__device__ __forceinline__ void swap16(uint32_t& a, uint32_t& b) {
  const auto v = __builtin_amdgcn_permlane16_swap(a, b, false, false);
  a = v[0];
  b = v[1];
}
__device__ __forceinline__ void swap32(uint32_t& a, uint32_t& b) {
  const auto v = __builtin_amdgcn_permlane32_swap(a, b, false, false);
  a = v[0];
  b = v[1];
}
// Lane (r, kq) holds the fp16 scales of groups 4kq..4kq+3 of its weight row
// (2 dwords); afterwards d[u] holds the scale of group 4u + kq, duplicated
// into both halves of the dword (a 4x4 transpose over the row's 4 lanes).
__device__ __forceinline__ void transpose_scales(uint32_t lo, uint32_t hi, uint32_t (&d)[4]) {
  d[0] = __builtin_amdgcn_perm(hi, lo, 0x01000100u);
  d[1] = __builtin_amdgcn_perm(hi, lo, 0x03020302u);
  d[2] = __builtin_amdgcn_perm(hi, lo, 0x05040504u);
  d[3] = __builtin_amdgcn_perm(hi, lo, 0x07060706u);
  swap16(d[0], d[1]);
  swap16(d[2], d[3]);
  swap32(d[0], d[2]);
  swap32(d[1], d[3]);
}
// The same transpose, kept two scales to a dword: c[0] holds the scales of
// sub-steps 0 and 1 (low and high half), c[1] those of sub-steps 2 and 3.
__device__ __forceinline__ void transpose_scales_c(uint32_t lo, uint32_t hi, uint32_t (&c)[2]) {
  uint32_t d[4];
  transpose_scales(lo, hi, d);
  c[0] = __builtin_amdgcn_perm(d[1], d[0], 0x05040100u);
  c[1] = __builtin_amdgcn_perm(d[3], d[2], 0x05040100u);
}
// The fp16 scale of sub-step u, in both halves of a dword: from the compact
// form (two to a dword) or the plain one (one per dword, already doubled).
__device__ __forceinline__ uint32_t scale_of(const uint32_t (&c)[2], int u) {
  return __builtin_amdgcn_perm(c[u >> 1], c[u >> 1], (u & 1) ? 0x03020302u : 0x01000100u);
}
__device__ __forceinline__ uint32_t scale_of(const uint32_t (&c)[4], int u) { return c[u]; }
__device__ __forceinline__ void transpose_scales_to(uint32_t lo, uint32_t hi, uint32_t (&c)[2]) {
  transpose_scales_c(lo, hi, c);
}
__device__ __forceinline__ void transpose_scales_to(uint32_t lo, uint32_t hi, uint32_t (&d)[4]) {
  transpose_scales(lo, hi, d);
}

// Raw buffer resource over [base, base + bytes): loads take a 32-bit per-lane
// offset and a scalar per-step offset, and read 0 past the end.
__device__ __forceinline__ __amdgpu_buffer_rsrc_t buffer_rsrc(const void* base, uint32_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0, (int)bytes, 0x00020000);
}
// 16 bytes per lane from a raw buffer straight into LDS: lane l's bytes
// land at lds + 16*l (lds is wave-uniform); out-of-range lanes write zeros.
// Kept out of the kernel templates, whose host-side instantiation cannot
// take this builtin.
__device__ __forceinline__ void load_lds16(__amdgpu_buffer_rsrc_t r, _Float16* lds, uint32_t voff, uint32_t soff) {
  __builtin_amdgcn_raw_ptr_buffer_load_lds(r, (__attribute__((address_space(3))) void*)lds, 16, voff, soff, 0, 0);
}
// Wait until at most N vector-memory loads of this wave are outstanding
// (expcnt and lgkmcnt left free; the gfx9 s_waitcnt field layout).
template <int N>
__device__ __forceinline__ void wait_vmcnt() {
  static_assert(N >= 0 && N < 64, "vmcnt is 6 bits");
  __builtin_amdgcn_s_waitcnt((N & 15) | (7 << 4) | (15 << 8) | ((N >> 4) << 14));
}
constexpr uint32_t kOob = 0x7FFFFF00u;  // a lane offset past any buffer: its loads read 0
constexpr int kSuper = 4 * kKStep;     // inputs per super-step (16 groups)

// 128-row tiles.  One work item = (expert, up to MB*16 routed rows) x (an N
// range).  A block has WN (4 or 8) waves along N, each NBW blocks of 16 output
// columns (gate+up: each with its up block).
//
// K is walked in super-steps of 512 inputs (16 groups of 32).  In sub-step
// u lane group kq (= lane/16) decodes group 4u + kq: the 16 code bytes at
// 64u + 16kq of the row's 256-byte chunk, which the codes' tile order
// (the layer's copy) puts at 16 * lane of the block's 1 KiB for the
// sub-step, so one load instruction reads 1 KiB contiguous.  The scales come from one 8-byte load per row and
// super-step (lane kq: groups 4kq..4kq+3) and a transpose across the row's
// four lanes.  The MFMA k-slot order is free as long as the activations
// follow it, so the activation fragment of sub-step u, MFMA i is inputs
// (4u+kq)*32 + 8i .. +8: in sub-step u the tile covers 256 contiguous
// bytes of each activation row.
// The block stages each sub-step's activation tile in LDS.
// Loads are buffer loads with a fixed per-lane offset and a scalar
// per-step offset (no vector address arithmetic); inputs past K read zeros.
template <int MB, int WN, int NBW, bool GATEUP>
__global__ __launch_bounds__(64 * WN) __attribute__((amdgpu_waves_per_eu(GATEUP ? kGuWPE : kDnWPE))) void gemm_kernel(GemmArgs g) {
  static_assert(WN == 4 || WN == 8, "4 or 8 waves along N");
  static_assert(MB > 1, "row tiles of at least 32 rows");
  constexpr int NBB = GATEUP ? 2 * NBW : NBW;
  const int tid = threadIdx.x, lane = tid & 63;
  // wave index as a wave-uniform (scalar) value, so loop bounds derived
  // from it give scalar branches and exact load counters
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int wn = wave;
  const int r = lane & 15, kq = lane >> 4;

  // all blocks of one item land on one XCD (block ids go round-robin over
  // 8), so the item's activation rows are reused from that XCD's L2
  const int bid = blockIdx.x, xcd = bid & 7, jj = bid >> 3;
  const int item = (jj / g.nblk) * 8 + xcd, nb = jj % g.nblk;
  // the item is read together with the item count (clamped into the list,
  // so both loads go out at once; a block past the count then returns)
  const int4 it = g.items[min(item, g.max_items - 1)];
  const int n_items = min(g.ctrl[g.count_at], g.max_items);
  if (item >= n_items) return;
  const int e = it.x, nr = it.z, pos0 = it.w;
  // work items come from the workspace: reject any that do not fit it
  if (e < 0 || e > g.E || nr <= 0 || nr > MB * 16 || pos0 < 0 || pos0 > g.R - nr) return;
  const uint32_t K2 = (uint32_t)g.K / 2, KG = (uint32_t)g.K / 32;
  const uint8_t* wb;
  const uint16_t* sbase;
  if (e < g.E) {
    wb = g.w + (size_t)e * g.Nw * K2;
    sbase = g.s + (size_t)e * g.Nw * KG;
  } else {
    if (g.w_sh == nullptr) return;
    wb = g.w_sh;
    sbase = g.s_sh;
  }
  const __amdgpu_buffer_rsrc_t rB = buffer_rsrc(wb, (uint32_t)g.Nw * K2);
  const __amdgpu_buffer_rsrc_t rS = buffer_rsrc(sbase, (uint32_t)g.Nw * KG * 2);
  const __amdgpu_buffer_rsrc_t rA = buffer_rsrc(g.a, g.a_bytes);

  // offsets of this lane's code chunk and scale quad within a 16-row B
  // block (vector; tile order: lane l's 16 bytes of a sub-step at 16 l of
  // the block's 1 KiB for it, its 8 bytes of scales of a super-step at 8 l
  // of the block's 512 bytes for it, so a load instruction reads 1 KiB or
  // 512 bytes contiguous), and each B block's first weight row
  // (wave-uniform, so it rides in the scalar offset; the lane part alone is
  // bounds-checked and every in-range lane stays inside the weights)
  const uint32_t tl = 16u * (uint32_t)lane, sl = 8u * (uint32_t)lane;
  uint32_t brow[NBB];
  int col0[NBW];
#pragma unroll
  for (int c = 0; c < NBW; ++c) {
    col0[c] = ((nb * WN + wn) * NBW + c) * 16;
    const uint32_t n0 = col0[c] < g.N ? col0[c] : 0;
    if (GATEUP) {
      brow[2 * c] = n0;
      brow[2 * c + 1] = g.N + n0;
    } else {
      brow[c] = n0;
    }
  }

  // super-steps: nss_full whole ones, then (if K % 512 != 0) one partial
  // with its missing groups masked
  const int nss_full = g.K / kSuper, nss = (g.K + kSuper - 1) / kSuper;
  const int S_begin = 0, S_end_full = nss_full;
  const bool has_tail = nss > nss_full;
  const int ngroups = g.K / 32;
  const int nmb = (nr + 15) / 16;

  float4_t acc[MB][NBB];
#pragma unroll
  for (int mb = 0; mb < MB; ++mb)
#pragma unroll
    for (int b = 0; b < NBB; ++b) acc[mb][b] = float4_t{0.f, 0.f, 0.f, 0.f};

  // codes of sub-step u of super-step S (ok: this lane's group exists)
  auto load_b = [&](int S, int u, Frag<NBB>& f, bool ok) __attribute__((always_inline)) {
#pragma unroll
    for (int b = 0; b < NBB; ++b)
      f.b[b] = __builtin_bit_cast(
          u32x4_t, __builtin_amdgcn_raw_buffer_load_b128(rB, ok ? tl + 1024u * u : kOob, S * (kSuper * 8) + brow[b] * K2, 0));
  };
  // the codes of sub-steps u and u + 1 of super-step S: per B block 2 KiB
  // contiguous in the tile order, issued back to back (in row order these
  // were the halves of each row's 128-byte line, served at the full
  // streaming rate when requested in adjacent instructions, a sub-step
  // apart at about 12% less on MI355X)
  auto load_b2 = [&](int S, int u, Frag<NBB>& f0, Frag<NBB>& f1, bool ok) __attribute__((always_inline)) {
#pragma unroll
    for (int b = 0; b < NBB; ++b) {
      f0.b[b] = __builtin_bit_cast(
          u32x4_t, __builtin_amdgcn_raw_buffer_load_b128(rB, ok ? tl + 1024u * u : kOob, S * (kSuper * 8) + brow[b] * K2, 0));
      f1.b[b] = __builtin_bit_cast(
          u32x4_t, __builtin_amdgcn_raw_buffer_load_b128(rB, ok ? tl + 1024u * (u + 1) : kOob, S * (kSuper * 8) + brow[b] * K2, 0));
    }
  };
  // the four scales of super-step S, as two dwords per B block
  auto load_sc = [&](int S, uint32_t (&sc)[NBB][2], bool ok) __attribute__((always_inline)) {
#pragma unroll
    for (int b = 0; b < NBB; ++b) {
      const auto v = __builtin_amdgcn_raw_buffer_load_b64(rS, ok ? sl : kOob, S * 512 + brow[b] * KG * 2, 0);
      sc[b][0] = v[0];
      sc[b][1] = v[1];
    }
  };
  // token of tile row m (m < nr), from its sorted slot; -1 if the slot is
  // not one of the call's
  auto tok_of = [&](int slot) __attribute__((always_inline)) -> int {
    if (slot < 0 || slot >= g.R) return -1;
    const int tok = slot < g.T ? slot / g.k : slot - g.T;
    return tok < g.M ? tok : -1;
  };

  // ---------------- prefill tiles: the activation tile of each sub-step
  // (MB*16 rows x 128 inputs) staged in LDS by direct global->LDS loads.
  // In sub-step u a row's inputs are four 64-byte segments (segment kq =
  // bytes 256u + 64kq of the row's super-step, the inputs of group 4u+kq).
  // One load instruction fills one LDS block of 1 KiB: rows q, q+4, q+8,
  // q+12 of a row block (lane l = 16rr + 4x + j takes byte 16j of the
  // segment stored at slot x of row q + 4rr), so every four lanes read 64
  // contiguous bytes.  Blocks are 1040 bytes apart.  In the down tiles
  // segment kq of row q + 4rr sits at slot (kq + 2rr + q) mod 4: the 16
  // lanes that read one MFMA operand column (rows 0..15, one segment, one
  // 16-byte piece) then meet no LDS bank conflict (measured on MI355X with
  // the LDS counters), down at 4096 tokens 12% faster.  Gate+up keeps slot
  // (kq + rr) mod 4 (4 conflict cycles per 8-cycle read): with the new slots
  // it measured up to 1% slower, so these reads do not bound it.  Wave w
  // loads block q = w mod 4 of every (WN/4)-th row block, starting at w / 4.
  constexpr int kBlkHalves = 520;  // 1040-byte LDS block
  // two buffers as separate arrays, so that the compiler can tell loads
  // into one from operand reads of the other
  __shared__ __attribute__((aligned(16))) _Float16 lds_a0[MB * 4 * kBlkHalves];
  __shared__ __attribute__((aligned(16))) _Float16 lds_a1[MB * 4 * kBlkHalves];
#define QMOE_LDS_A(BUF) ((BUF) ? lds_a1 : lds_a0)
  // Scales: this super-step's by sub-step (sc_cur), the next one's in load
  // layout (sc_nxt).  Gate+up, whose 8-block loop holds 128 accumulators,
  // keeps sc_cur two to a dword.
  constexpr bool kCompactSc = GATEUP;
  uint32_t sc_cur[NBB][kCompactSc ? 2 : 4], sc_nxt[NBB][2];
  Frag<NBB> fb0, fb1, fb2, fb3;  // the weights of sub-steps 0..3
  // Down: the first weights go out before the item's rows are looked up,
  // so the round trips of the lookups (sorted slot, routing weight) overlap
  // theirs instead of preceding them.  (Gate+up issues them after: its
  // 128 accumulators leave no room to hold them across the lookups.)
  // (down tiles of one 16-column block per wave only: wider waves have no
  // registers to hold these fragments across the lookups)
  constexpr bool kEarlyB = !GATEUP && NBW == 1;
  // (a K of only a partial super-step: the tail's first scales and weights)
  const bool early_tail = kEarlyB && S_end_full == S_begin && has_tail;
  if (kEarlyB && S_end_full > S_begin) {
    load_sc(S_begin, sc_nxt, true);
    load_b(S_begin, 0, fb0, true);
    load_b(S_begin, 1, fb1, true);
  } else if (early_tail) {
    load_sc(nss_full, sc_nxt, nss_full * 16 + 4 * kq < ngroups);
    load_b(nss_full, 0, fb0, nss_full * 16 + kq < ngroups);
    if (nss_full * 16 + 4 < ngroups) load_b(nss_full, 1, fb1, nss_full * 16 + 4 + kq < ngroups);
  }
  // per tile row: activation offset and the token's scale, read by the
  // epilogue (gate+up: 2^e, which takes x's scaling off g and u; down: its
  // slot, and the routing weight times 2^2e, which takes h's scaling off)
  __shared__ uint32_t lds_row[MB * 16];
  __shared__ float lds_sc[MB * 16];
  __shared__ int lds_slot[GATEUP ? 1 : MB * 16];
  for (int m = tid; m < MB * 16; m += 64 * WN) {
    const int slot = m < nr ? g.perm[pos0 + m] : -1;
    const int tok = tok_of(slot);
    const int e = tok >= 0 ? g.xexp[tok] : 0;
    if (GATEUP) {
      lds_row[m] = tok >= 0 ? (uint32_t)tok * (uint32_t)g.K * 2 : kOob;
      lds_sc[m] = pow2f(e);
    } else {
      lds_row[m] = m < nr ? (uint32_t)(pos0 + m) * (uint32_t)g.K * 2 : kOob;
      lds_slot[m] = slot;
      lds_sc[m] = ((slot >= 0 && slot < g.T) ? g.wts[slot] : 1.0f) * pow2f(2 * e);
    }
  }
  __syncthreads();
  // loads: per row block this wave loads, this lane's row (q = wave mod 4,
  // rr = lane/16) offset plus its segment and piece; rows past the item
  // read zeros
  constexpr int MBS = WN / 4, NA = MB / MBS;
  static_assert(MB % MBS == 0, "row blocks split evenly over the waves");
  const int aq = wave & 3, amb0 = wave >> 2;
  uint32_t aoffs[NA];
  // slot of segment kq of row q + 4rr: (kq + rr + kSlotQ * (rr + q)) mod 4
  constexpr int kSlotQ = GATEUP ? 0 : 1;
  const int aseg = (((lane >> 2) & 3) - (lane >> 4) - kSlotQ * ((lane >> 4) + aq)) & 3;  // the segment this lane loads
  {
    const uint32_t inrow = 64 * aseg + 16 * (lane & 3);
    const int rr = lane >> 4;
#pragma unroll
    for (int t = 0; t < NA; ++t) {
      const uint32_t o = lds_row[(amb0 + MBS * t) * 16 + aq + 4 * rr];
      aoffs[t] = o == kOob ? kOob : o + inrow;
    }
  }
  // operand reads: lane (r, kq) reads row r = q + 4rr, segment kq, piece i
  const int rd_half =
      (r & 3) * kBlkHalves + 128 * (r >> 2) + 32 * ((kq + (r >> 2) + kSlotQ * ((r >> 2) + (r & 3))) & 3);
  auto promote_scales = [&]() __attribute__((always_inline)) {
#pragma unroll
    for (int b = 0; b < NBB; ++b) transpose_scales_to(sc_nxt[b][0], sc_nxt[b][1], sc_cur[b]);
  };
  // this wave's blocks of sub-step U of super-step S into buffer BUF, for
  // the NMBC row blocks in use (row block amb0 + MBS*t; a wave-uniform
  // test); lanes whose group is past K (OK false) read zeros
#define QMOE_LOAD_A_TILE_AT(S, U, OK, BUF, SLOT0)                                                \
  do {                                                                                           \
    _Pragma("unroll") for (int t = 0; t < NA; ++t) {                                             \
      if (MBS == 1 ? t < NMBC : amb0 + MBS * t < NMBC)                                           \
        load_lds16(rA, &QMOE_LDS_A(BUF)[(((SLOT0) + amb0 + MBS * t) * 4 + aq) * kBlkHalves],      \
                   (OK) ? aoffs[t] : kOob, (S) * (kSuper * 2) + 256 * (U));                      \
    }                                                                                            \
  } while (0)
#define QMOE_LOAD_A_TILE(S, U, OK, BUF) QMOE_LOAD_A_TILE_AT(S, U, OK, BUF, 0)
#define QMOE_COMPUTE(F, SC, U, BUF) QMOE_COMPUTE_AT(F, SC, U, BUF, 0)
#define QMOE_COMPUTE_AT(F, SC, U, BUF, SLOT0)                                                    \
  do {                                                                                           \
    uint32_t s2_[NBB];                                                                           \
    _Pragma("unroll") for (int b = 0; b < NBB; ++b) s2_[b] = scale_of((SC)[b], (U));             \
    half8_t bfa_[NBB], bfb_[NBB];                                                                \
    _Pragma("unroll") for (int b = 0; b < NBB; ++b) bfa_[b] = dq8p(word((F).b[b], 0), s2_[b]);   \
    _Pragma("unroll") for (int i = 0; i < 4; ++i) {                                              \
      /* k-slice i's MFMAs, and the decode of slice i+1 in the same */                           \
      /* scheduling region so the two can interleave */                                          \
      half8_t* cur_ = (i & 1) ? bfb_ : bfa_;                                                     \
      half8_t* nxt_ = (i & 1) ? bfa_ : bfb_;                                                     \
      _Pragma("unroll") for (int mb = 0; mb < MB; ++mb) {                                        \
        if (mb < NMBC) {                                                                         \
          const half8_t av =                                                                     \
              *reinterpret_cast<const half8_t*>(&QMOE_LDS_A(BUF)[((SLOT0) + mb) * 4 * kBlkHalves + rd_half + 8 * i]); \
          _Pragma("unroll") for (int b = 0; b < NBB; ++b) acc[mb][b] = mfma16x16x32(av, cur_[b], acc[mb][b]); \
        }                                                                                        \
      }                                                                                          \
      if (i < 3) {                                                                               \
        _Pragma("unroll") for (int b = 0; b < NBB; ++b) nxt_[b] = dq8p(word((F).b[b], i + 1), s2_[b]); \
      }                                                                                          \
      /* 4 weight blocks: one slice at a time keeps their 128 accumulators */                    \
      /* within 256 registers */                                                                 \
      if (NBB >= 4) __builtin_amdgcn_sched_barrier(0);                                           \
    }                                                                                            \
  } while (0)
  // The same compute with the weights of the sub-step after next issued one
  // 16-row block per k-slice (block b before slice b mod 4) instead of all
  // before the compute: a wave whose load waits for room in the address
  // unit's queue then still has MFMAs of the slices before it issued (gate+up
  // at 4096 tokens 3% faster on MI355X).
#define QMOE_COMPUTE_IL(F, SC, U, BUF, SB, UB, FNN)                                               \
  do {                                                                                           \
    uint32_t s2_[NBB];                                                                           \
    _Pragma("unroll") for (int b = 0; b < NBB; ++b) s2_[b] = scale_of((SC)[b], (U));             \
    half8_t bfa_[NBB], bfb_[NBB];                                                                \
    _Pragma("unroll") for (int b = 0; b < NBB; ++b) bfa_[b] = dq8p(word((F).b[b], 0), s2_[b]);   \
    _Pragma("unroll") for (int i = 0; i < 4; ++i) {                                              \
      _Pragma("unroll") for (int b = 0; b < NBB; ++b) {                                          \
        if (b % 4 == i)                                                                          \
          (FNN).b[b] = __builtin_bit_cast(u32x4_t, __builtin_amdgcn_raw_buffer_load_b128(        \
              rB, tl + 1024u * (UB), (SB) * (kSuper * 8) + brow[b] * K2, 0));                       \
      }                                                                                          \
      half8_t* cur_ = (i & 1) ? bfb_ : bfa_;                                                     \
      half8_t* nxt_ = (i & 1) ? bfa_ : bfb_;                                                     \
      _Pragma("unroll") for (int mb = 0; mb < MB; ++mb) {                                        \
        if (mb < NMBC) {                                                                         \
          const half8_t av =                                                                     \
              *reinterpret_cast<const half8_t*>(&QMOE_LDS_A(BUF)[mb * 4 * kBlkHalves + rd_half + 8 * i]); \
          _Pragma("unroll") for (int b = 0; b < NBB; ++b) acc[mb][b] = mfma16x16x32(av, cur_[b], acc[mb][b]); \
        }                                                                                        \
      }                                                                                          \
      if (i < 3) {                                                                               \
        _Pragma("unroll") for (int b = 0; b < NBB; ++b) nxt_[b] = dq8p(word((F).b[b], i + 1), s2_[b]); \
      }                                                                                          \
      __builtin_amdgcn_sched_barrier(0);                                                         \
    }                                                                                            \
  } while (0)
  // One sub-step with one barrier: start the next sub-step's activation
  // tile (into the other buffer) and, spread over the k-slices, the weights
  // of the sub-step after next (into FNN), compute this sub-step from
  // fragment set FCUR and
  // buffer BUF, then wait until at most the NBB weight loads just issued
  // are outstanding (loads complete in order, so the tile, written straight
  // into LDS, and the next sub-step's weights are in) and meet the barrier
  // that publishes the tile and frees BUF.  Weights get two sub-steps to
  // arrive, the activation tile one.
#define QMOE_SUBSTEP(U, FCUR, SA, UA, SB, UB, FNN, BUF)                                         \
  do {                                                                                           \
    QMOE_LOAD_A_TILE((SA), (UA), true, (BUF) ^ 1);                                               \
    __builtin_amdgcn_sched_barrier(0); /* keep the tile loads ahead of the compute */            \
    QMOE_COMPUTE_IL(FCUR, sc_cur, (U), (BUF), (SB), (UB), FNN);                                  \
    wait_vmcnt<NBB>();                                                                           \
    __syncthreads();                                                                             \
  } while (0)
  // The same with the weights of the two sub-steps after next issued as
  // pairs (FN0, FN1), or with no weights (a sub-step whose pair
  // went out with the previous one's).  All loads are waited for except the
  // pair just issued.
#define QMOE_SUBSTEP_PAIR(U, FCUR, SA, UA, SB, UB, FN0, FN1, BUF)                               \
  do {                                                                                           \
    QMOE_LOAD_A_TILE((SA), (UA), true, (BUF) ^ 1);                                               \
    load_b2((SB), (UB), FN0, FN1, true);                                                         \
    __builtin_amdgcn_sched_barrier(0);                                                           \
    QMOE_COMPUTE(FCUR, sc_cur, (U), (BUF));                                                      \
    wait_vmcnt<2 * NBB>();                                                                       \
    __syncthreads();                                                                             \
  } while (0)
#define QMOE_SUBSTEP_NOB(U, FCUR, SA, UA, BUF)                                                  \
  do {                                                                                           \
    QMOE_LOAD_A_TILE((SA), (UA), true, (BUF) ^ 1);                                               \
    __builtin_amdgcn_sched_barrier(0);                                                           \
    QMOE_COMPUTE(FCUR, sc_cur, (U), (BUF));                                                      \
    wait_vmcnt<0>();                                                                             \
    __syncthreads();                                                                             \
  } while (0)
  // The partial super-step (K % 512 != 0; groups past K read zeros): its
  // sub-steps go two at a time, one per LDS buffer, their weights, tiles
  // and (with the first pair) the scales behind one wait, so a 256-input K
  // (one GPU's share of an 8-way tensor-parallel down product, all tail)
  // costs one trip to memory instead of three.  K is a multiple of 128, so a
  // lane's four scales lie in the row or all past it; only the lane offset
  // is range-checked, so lanes past the row must not read.
#define QMOE_TAIL()                                                                              \
  do {                                                                                           \
    _Pragma("unroll") for (int u0 = 0; u0 < 4; u0 += 2) {                                        \
      if (nss_full * 16 + 4 * u0 >= ngroups) break; /* sub-steps wholly past K (wave-uniform) */ \
      const bool two_ = nss_full * 16 + 4 * (u0 + 1) < ngroups;                                  \
      __syncthreads(); /* every wave is done reading both buffers */                             \
      if (!(u0 == 0 && early_tail)) { /* (else already in flight) */                             \
        if (u0 == 0) load_sc(nss_full, sc_nxt, nss_full * 16 + 4 * kq < ngroups);                 \
        load_b(nss_full, u0, fb0, nss_full * 16 + 4 * u0 + kq < ngroups);                        \
        if (two_) load_b(nss_full, u0 + 1, fb1, nss_full * 16 + 4 * (u0 + 1) + kq < ngroups);    \
      }                                                                                          \
      QMOE_LOAD_A_TILE(nss_full, u0, nss_full * 16 + 4 * u0 + aseg < ngroups, 0);                 \
      if (two_) QMOE_LOAD_A_TILE(nss_full, u0 + 1, nss_full * 16 + 4 * (u0 + 1) + aseg < ngroups, 1); \
      __builtin_amdgcn_s_waitcnt(0);                                                             \
      __syncthreads();                                                                           \
      if (u0 == 0) promote_scales();                                                             \
      QMOE_COMPUTE(fb0, sc_cur, u0, 0);                                                          \
      if (two_) QMOE_COMPUTE(fb1, sc_cur, u0 + 1, 1);                                            \
    }                                                                                            \
  } while (0)
  // The row blocks that hold routed rows are computed without a branch per
  // block: the loop is instantiated for 2, 4, 5, 6, 7 and 8 blocks (about
  // 85 rows per expert at 4096 tokens: 5-7 blocks) and the item's count
  // rounds up to the next of these (blocks past the item's rows multiply
  // zero rows, which are never stored).
  auto kloop = [&](auto nmbc_tag) __attribute__((always_inline)) {
    constexpr int NMBC = decltype(nmbc_tag)::value;
    const int n = S_end_full - S_begin;
    if (n > 0) {
      if (!kEarlyB) {
        load_sc(S_begin, sc_nxt, true);
        load_b(S_begin, 0, fb0, true);
        QMOE_LOAD_A_TILE(S_begin, 0, true, 0);
        load_b(S_begin, 1, fb1, true);
        wait_vmcnt<NBB>();
      } else {  // the first two sub-steps' weights are already in flight
        QMOE_LOAD_A_TILE(S_begin, 0, true, 0);
        wait_vmcnt<0>();
      }
      __syncthreads();
      promote_scales();
      for (int S = S_begin; S < S_end_full; ++S) {
        // the next super-step, clamped: the last one reloads itself
        const int Sn = min(S + 1, S_end_full - 1);
        if constexpr (GATEUP && NMBC <= kGuPairRowBlocks) {
          // weights two sub-steps at a time: sub-steps 2 and 3 go out with
          // sub-step 0, the next super-step's 0 and 1 with sub-step 2.  The
          // next scales go out with sub-step 3's tile, whose deadline they
          // share: held from there to their use they take no registers
          // through the other sub-steps
          QMOE_SUBSTEP_PAIR(0, fb0, S, 1, S, 2, fb2, fb3, 0);
          QMOE_SUBSTEP_NOB(1, fb1, S, 2, 1);
          QMOE_SUBSTEP_PAIR(2, fb2, S, 3, Sn, 0, fb0, fb1, 0);
          load_sc(Sn, sc_nxt, true);
          QMOE_SUBSTEP_NOB(3, fb3, Sn, 0, 1);
        } else {
          load_sc(Sn, sc_nxt, true);
          QMOE_SUBSTEP(0, fb0, S, 1, S, 2, fb2, 0);
          QMOE_SUBSTEP(1, fb1, S, 2, S, 3, fb3, 1);
          QMOE_SUBSTEP(2, fb2, S, 3, Sn, 0, fb0, 0);
          QMOE_SUBSTEP(3, fb3, Sn, 0, Sn, 1, fb1, 1);
        }
        promote_scales();
      }
    }
    if (has_tail) QMOE_TAIL();
  };
  // Down items of at most 32 rows: a whole super-step of their activation
  // tile (4 sub-steps x 2 row blocks) fits one buffer, so the block loads
  // the next super-step's tile and weights at once, one super-step ahead,
  // and meets one barrier per super-step instead of one per sub-step.  With
  // so few rows a sub-step is only 8 MFMAs per wave, far shorter than a trip
  // to memory; this doubles the bytes each wave keeps in flight.
  auto kloop_ss = [&](auto) __attribute__((always_inline)) {  // (generic: instantiated only where used)
    constexpr int NMBC = 2;
    static_assert(MB >= 4 * NMBC, "a super-step of 2-block tiles fits one buffer");
    Frag<NBB> fc0, fc1, fc2, fc3;  // the other super-step's weights
    if (S_end_full > S_begin) {
      // fb0, fb1 and the scales of the first super-step are in flight
      load_b(S_begin, 2, fb2, true);
      load_b(S_begin, 3, fb3, true);
#pragma unroll
      for (int u = 0; u < 4; ++u) QMOE_LOAD_A_TILE_AT(S_begin, u, true, 0, u * NMBC);
      wait_vmcnt<0>();
      __syncthreads();
      promote_scales();
      for (int S = S_begin; S < S_end_full; S += 2) {
        // super-step S from buffer 0 and fb*, while S + 1 comes into
        // buffer 1 and fc* (past the range every lane reads zeros)
        const bool more1 = S + 1 < S_end_full;
        load_sc(S + 1, sc_nxt, more1);
#pragma unroll
        for (int u = 0; u < 4; ++u) QMOE_LOAD_A_TILE_AT(S + 1, u, more1, 1, u * NMBC);
        load_b(S + 1, 0, fc0, more1);
        load_b(S + 1, 1, fc1, more1);
        load_b(S + 1, 2, fc2, more1);
        load_b(S + 1, 3, fc3, more1);
        __builtin_amdgcn_sched_barrier(0);
        QMOE_COMPUTE_AT(fb0, sc_cur, 0, 0, 0 * NMBC);
        QMOE_COMPUTE_AT(fb1, sc_cur, 1, 0, 1 * NMBC);
        QMOE_COMPUTE_AT(fb2, sc_cur, 2, 0, 2 * NMBC);
        QMOE_COMPUTE_AT(fb3, sc_cur, 3, 0, 3 * NMBC);
        wait_vmcnt<0>();
        __syncthreads();
        if (!more1) break;
        promote_scales();
        // super-step S + 1 from buffer 1 and fc*, while S + 2 comes into
        // buffer 0 and fb*
        const bool more2 = S + 2 < S_end_full;
        load_sc(S + 2, sc_nxt, more2);
#pragma unroll
        for (int u = 0; u < 4; ++u) QMOE_LOAD_A_TILE_AT(S + 2, u, more2, 0, u * NMBC);
        load_b(S + 2, 0, fb0, more2);
        load_b(S + 2, 1, fb1, more2);
        load_b(S + 2, 2, fb2, more2);
        load_b(S + 2, 3, fb3, more2);
        __builtin_amdgcn_sched_barrier(0);
        QMOE_COMPUTE_AT(fc0, sc_cur, 0, 1, 0 * NMBC);
        QMOE_COMPUTE_AT(fc1, sc_cur, 1, 1, 1 * NMBC);
        QMOE_COMPUTE_AT(fc2, sc_cur, 2, 1, 2 * NMBC);
        QMOE_COMPUTE_AT(fc3, sc_cur, 3, 1, 3 * NMBC);
        wait_vmcnt<0>();
        __syncthreads();
        promote_scales();
      }
    }
    if (has_tail) QMOE_TAIL();
  };
  // ---- epilogue: lane holds rows mb*16 + 4*kq + i of column r of each
  // block.  It runs inside each row-block instance (NMBC blocks), so an
  // instance keeps only its own blocks' accumulators live through its K loop.
  auto epilogue = [&](auto nmbc_tag) __attribute__((always_inline)) {
    constexpr int NMBC = decltype(nmbc_tag)::value;
#pragma unroll
    for (int c = 0; c < NBW; ++c) {
      if (col0[c] >= g.N) continue;
      const int col = col0[c] + r;
#pragma unroll
      for (int mb = 0; mb < NMBC; ++mb) {
        if (mb >= nmb) continue;
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const int row = mb * 16 + 4 * kq + i;
          if (row >= nr) continue;
          const int pos = pos0 + row;
          if (GATEUP) {
            // g = acc * 2^e; h is stored times 2^-2e: SiLU(g) * (acc_up * 2^-e),
            // odd columns divided by 16 (operand format)
            const float sc = lds_sc[row];
            const float gt = acc[mb][2 * c][i] * sc;
            const float up = acc[mb][2 * c + 1][i] * inv_pow2f(sc) * ((col & 1) ? 0.0625f : 1.0f);
            g.h_out[(size_t)pos * g.N + ((col & ~7) | inv_perm8(col & 7))] = silu_mul_h(gt, up);
          } else {
            const int slot = lds_slot[row];
            if (slot < 0 || slot >= g.R) continue;
            g.y_out[(size_t)slot * g.N + col] = (uint16_t)f32_to_bf16_rne(lds_sc[row] * acc[mb][c][i]);
          }
        }
      }
    }
  };
  auto body = [&](auto nmbc_tag) __attribute__((always_inline)) {
    kloop(nmbc_tag);
    epilogue(nmbc_tag);
  };
  if (nmb <= 2) {
    if constexpr (kEarlyB && MB >= 8) {
      kloop_ss(0);
      epilogue(std::integral_constant<int, 2>{});
    } else {
      body(std::integral_constant<int, (MB < 2 ? MB : 2)>{});
    }
  } else if (nmb <= 4) body(std::integral_constant<int, (MB < 4 ? MB : 4)>{});
  else if (MB == 8 && nmb == 5) body(std::integral_constant<int, 5>{});
  else if (nmb <= 6) body(std::integral_constant<int, (MB < 6 ? MB : 6)>{});
  else if (MB == 8 && nmb == 7) body(std::integral_constant<int, 7>{});
  else body(std::integral_constant<int, MB>{});
#undef QMOE_SUBSTEP
#undef QMOE_TAIL
#undef QMOE_COMPUTE_IL
#undef QMOE_SUBSTEP_PAIR
#undef QMOE_SUBSTEP_NOB
#undef QMOE_COMPUTE
#undef QMOE_COMPUTE_AT
#undef QMOE_LOAD_A_TILE
#undef QMOE_LOAD_A_TILE_AT
#undef QMOE_LDS_A
}

// -------------------------------------------------------- GEMV (1-2 rows)

// Work items of at most kGemvRows routed rows, used while a call averages
// at most 1.75 routed rows per expert (small M).  There each expert's
// product is a weight-streaming matrix-vector product, so it runs on packed
// fp16 dot products (v_dot2_f32_f16) rather than MFMA tiles: on MI355X,
// MFMAs fed from a full-rate weight stream hold back the stream's load
// issue, while the dot-product form keeps it close to the read bandwidth.
//
// K is walked in super-steps of 512 inputs: a 256-byte chunk of each
// weight row, 16 groups of 32.  Lane (q, j) of a wave (q = lane/16) takes
// group j of every super-step, for rows 4m + q (m = 0..3) of each 16-row
// weight block, so one load instruction reads four whole 256-byte chunks
// (eight full cache lines) of the codes as the caller gave them, in row
// order (the MFMA tiles read the layer's tile-order copy instead: in that
// order these loads would read 64-byte halves of 16 lines, which measured
// 15-27% slower), and a lane reads its group's activations once per
// super-step for all of its rows.  Each lane loads its group's scale
// per row.  The 16 lanes of a row hold partial sums over different groups;
// a butterfly over those lanes adds them once, after the K loop.
//
// Arithmetic: a nibble q masked in place is read as an fp16 bit pattern,
// the subnormal q * 2^-24 (for the odd inputs, whose nibble sits 4 bits up,
// 16q * 2^-24, and their activations are stored divided by 16), so the
// decode is one AND per pair of codes.  Dot products with the activations
// give 2^-24 * sum(x*q) in fp32 (exact products); the zero point comes back
// as 8 * sum(x) per group, computed once per staged row, and the group's
// scale multiplies 2^24 * p - 8 * sum(x) in fp32.
//
// The item's activation rows are staged in LDS once per block, each
// group's 64 bytes padded to 80 so that the 16 groups a wave reads at once
// fall in distinct banks; the padding holds the group's 8 * sum(x).
constexpr int kGemvRows = 2;
constexpr int kGemvMaxRowsPer4Experts = 7;  // GEMV while 4*M*top_k <= 7E
constexpr int kGemvGroupBytes = 80;         // one staged group of 32 fp16 inputs, padded
constexpr int kGemvMaxK = 13056;            // largest K the GEMV stages (two rows in 64 KiB of LDS)

// LDS bytes of a block: the activation rows
__host__ __device__ constexpr size_t gemv_lds_bytes(int K) {
  return (size_t)kGemvRows * (K / 32) * kGemvGroupBytes;
}

// Three waves per SIMD: the ping-pong of whole super-steps holds 80 registers
// of weights, and each per-row-count instance of the body fits in 168
// registers without spills (capped at four waves it spills inside the K
// loop).  Measured on MI355X against two waves: the 9-token call 281 -> 269
// us, the I=256 slice at one token 35.3 -> 30.5 us.  A deeper ring of
// super-steps per wave (three or four in flight, two waves) measured 4-12%
// slower than more waves with two in flight.
constexpr int kGemvWPE = 3;
// NT: weight codes are read with the non-temporal cache policy.  A plain
// streaming read measured about 6.7 TB/s that way against 6.2 TB/s with the
// default policy on MI355X; it pays only while each expert's codes are read
// once (about one routed row per expert or fewer).  Scales keep the default
// policy (non-temporal scales measured slower at every M).
template <bool GATEUP, bool NT>
__global__ __launch_bounds__(kThreads) __attribute__((amdgpu_waves_per_eu(kGemvWPE))) void gemv_kernel(
    GemmArgs g) {
  constexpr int WN = kThreads / 64;      // waves along N
  constexpr int NBB = 2;                 // weight blocks of 16 rows per wave
  constexpr int NBW = GATEUP ? 1 : 2;    // output column blocks per wave
  const int tid = threadIdx.x, lane = tid & 63;
  const int wn = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int q = lane >> 4, j = lane & 15;

  // consecutive blocks take consecutive column blocks of one item, so each
  // item's stream is spread over all XCDs
  // (split-K: the grid holds `splits` copies of that, split s taking the
  // s-th share of K)
  const int per_split = g.nblk * g.max_items;
  const int split = (int)blockIdx.x / per_split, local = (int)blockIdx.x % per_split;
  const int item = local / g.nblk, nb = local % g.nblk;
  // the item is read together with the item count (clamped into the list,
  // so both loads go out at once; a block past the count then returns)
  const int4 it = g.items[min(item, g.max_items - 1)];
  const int n_items = min(g.ctrl[g.count_at], g.max_items);
  if (item >= n_items) return;
  const int e = it.x, nr = it.z, pos0 = it.w;
  if (e < 0 || e > g.E || nr <= 0 || nr > kGemvRows || pos0 < 0 || pos0 > g.R - nr) return;
  const uint32_t K2 = (uint32_t)g.K / 2, KG = (uint32_t)g.K / 32;
  const uint8_t* wb;
  const uint16_t* sbase;
  if (e < g.E) {
    wb = g.w + (size_t)e * g.Nw * K2;
    sbase = g.s + (size_t)e * g.Nw * KG;
  } else {
    if (g.w_sh == nullptr) return;
    wb = g.w_sh;
    sbase = g.s_sh;
  }
  const __amdgpu_buffer_rsrc_t rB = buffer_rsrc(wb, (uint32_t)g.Nw * K2);
  const __amdgpu_buffer_rsrc_t rS = buffer_rsrc(sbase, (uint32_t)g.Nw * KG * 2);
  const __amdgpu_buffer_rsrc_t rA = buffer_rsrc(g.a, g.a_bytes);

  // lane part of the code and scale offsets (row q, group j; the codes as
  // the caller gave them, in row order), and each block's first weight row
  // (wave-uniform, in the scalar offset; every in-range lane stays inside
  // the weights)
  const uint32_t bl = (uint32_t)q * K2 + 16 * j, sl = (uint32_t)q * KG * 2 + 2 * j;
  uint32_t brow[NBB];
  int col0[NBW];
#pragma unroll
  for (int c = 0; c < NBW; ++c) {
    col0[c] = ((nb * WN + wn) * NBW + c) * 16;
    const uint32_t n0 = col0[c] < g.N ? col0[c] : 0;
    if (GATEUP) {  // gate rows n0.. and up rows N + n0..
      brow[0] = n0;
      brow[1] = g.N + n0;
    } else {
      brow[c] = n0;
    }
  }

  const int nss_full = g.K / kSuper, nss = (g.K + kSuper - 1) / kSuper;
  const int S_begin = split * nss / g.splits, S_end = (split + 1) * nss / g.splits;
  const int S_end_full = min(S_end, nss_full);
  const bool has_tail = S_end > nss_full;  // the partial super-step (last split only)
  const int ngroups = g.K / 32;

  // one super-step of this lane's weights: group j of rows 4m + q of each
  // block (16 code bytes and the fp16 scale each)
  struct Super {
    u32x4_t b[NBB][4];
    uint32_t sc[NBB][4];
  };
  // ok: this lane's group exists (false: codes and scale read 0)
  auto load_super = [&](int S, Super& f, bool ok) __attribute__((always_inline)) {
#pragma unroll
    for (int m = 0; m < 4; ++m)
#pragma unroll
      for (int b = 0; b < NBB; ++b)
        f.b[b][m] = __builtin_bit_cast(
            u32x4_t, __builtin_amdgcn_raw_buffer_load_b128(rB, ok ? bl : kOob,
                                                           (brow[b] + 4 * m) * K2 + S * (kSuper / 2), NT ? 2 : 0));
#pragma unroll
    for (int m = 0; m < 4; ++m)
#pragma unroll
      for (int b = 0; b < NBB; ++b)
        f.sc[b][m] = __builtin_amdgcn_raw_buffer_load_b16(rS, ok ? sl : kOob, (brow[b] + 4 * m) * KG * 2 + S * 32, 0);
  };

  // Everything from here on is instantiated per row count of the item (1 or
  // 2), so each instance is register-allocated on its own (one-row items do
  // not carry the second row's lookups, activations and sums).
  auto path = [&](auto rows_tag) __attribute__((always_inline)) {
    constexpr int NR = decltype(rows_tag)::value;
    // the first super-step's loads go out before the rows are staged
    Super fa, fb;
    if (S_end_full > S_begin) load_super(S_begin, fa, true);
    // each row's slot, token and scale are read now, so their dependent round
    // trips overlap the weight stream instead of following it.  Gate+up: 2^e
    // (x rows are held times 2^-e); down: the routing weight times 2^2e (h
    // rows are held times 2^-2e)
    int slot_of[NR], tok_of[NR];
    float sc_of[NR];
#pragma unroll
    for (int t = 0; t < NR; ++t) {
      const int sl = t < nr ? g.perm[pos0 + t] : -1;
      const int tok = (sl >= 0 && sl < g.R) ? (sl < g.T ? sl / g.k : sl - g.T) : -1;
      slot_of[t] = sl;
      tok_of[t] = tok < g.M ? tok : -1;
    }
#pragma unroll
    for (int t = 0; t < NR; ++t) {
      const int e = tok_of[t] >= 0 ? g.xexp[tok_of[t]] : 0;
      const int sl = slot_of[t];
      sc_of[t] = GATEUP ? pow2f(e) : ((sl >= 0 && sl < g.T) ? g.wts[sl] : 1.0f) * pow2f(2 * e);
    }

    // ---- stage the item's activation rows (operand format) in LDS: group
    // gi's four 16-byte runs at gi * 80 bytes
    extern __shared__ __attribute__((aligned(16))) uint32_t gemv_lds[];
    u32x4_t* lds_x = reinterpret_cast<u32x4_t*>(gemv_lds);
    constexpr int kGroupRuns = kGemvGroupBytes / 16;  // 5: 4 runs + 1 of padding
    const int runs = g.K / 8;
    // (only this split's super-steps: runs [v_lo, v_hi))
    const int v_lo = S_begin * (kSuper / 8), v_hi = min(S_end * (kSuper / 8), runs);
    // and the group's code offset 8 * sum(x) as fp32 in the first word of its
    // padding (the four runs of a group sit in four adjacent lanes)
    for (int t = 0; t < nr; ++t) {
      uint32_t off;
      if (GATEUP) {
        off = tok_of[t] >= 0 ? (uint32_t)tok_of[t] * (uint32_t)g.K * 2 : kOob;
      } else {
        off = (uint32_t)(pos0 + t) * (uint32_t)g.K * 2;
      }
      for (int v0 = v_lo; v0 < v_hi; v0 += kThreads) {  // v_lo, v_hi multiples of 4: groups stay whole
        const int v = v0 + tid;
        const bool in = v < v_hi;
        const u32x4_t xr = __builtin_bit_cast(
            u32x4_t, __builtin_amdgcn_raw_buffer_load_b128(rA, (off == kOob || !in) ? kOob : off + 16 * v, 0, 0));
        float sx = 0.f;  // sum of the run's 8 inputs (positions 2, 3, 6, 7 are stored divided by 16)
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const half2_t hv = as_half2(xr[i]);
          sx += ((i & 1) ? 16.f : 1.f) * ((float)hv[0] + (float)hv[1]);
        }
        sx += __shfl_xor(sx, 1, 64);
        sx += __shfl_xor(sx, 2, 64);
        if (in) {
          u32x4_t* grp = lds_x + (t * ngroups + (v >> 2)) * kGroupRuns;
          grp[v & 3] = xr;
          if ((v & 3) == 0) reinterpret_cast<float*>(grp + 4)[0] = 8.f * sx;
        }
      }
    }
    __syncthreads();

    float acc[NBB][4][NR];
#pragma unroll
    for (int b = 0; b < NBB; ++b)
#pragma unroll
      for (int m = 0; m < 4; ++m)
#pragma unroll
        for (int t = 0; t < NR; ++t) acc[b][m][t] = 0.f;

    // Super-step S from registers.  A group past K (partial last super-step)
    // has scale 0 and reads the row's last group, so it adds exactly zero.
    auto compute_super = [&](int S, const Super& f) __attribute__((always_inline)) {
      const int gi = min(S * 16 + j, ngroups - 1);
      u32x4_t xv[NR][4];
      float cx[NR];  // 8 * sum(x) of the group
#pragma unroll
      for (int t = 0; t < NR; ++t) {
#pragma unroll
        for (int i = 0; i < 4; ++i) xv[t][i] = lds_x[(t * ngroups + gi) * kGroupRuns + i];
        cx[t] = reinterpret_cast<const float*>(lds_x + (t * ngroups + gi) * kGroupRuns + 4)[0];
      }
#pragma unroll
      for (int b = 0; b < NBB; ++b)
#pragma unroll
        for (int m = 0; m < 4; ++m) {
          float p[NR];
#pragma unroll
          for (int t = 0; t < NR; ++t) p[t] = 0.f;
#pragma unroll
          for (int i = 0; i < 4; ++i) {
            // the masked nibbles as fp16 bit patterns: q * 2^-24 (subnormal),
            // or 16q * 2^-24 for the odd inputs
            const uint32_t w = word(f.b[b][m], i), w8 = w >> 8;
            const half2_t w0 = as_half2(w & 0x000F000Fu);   // inputs 0, 4
            const half2_t w1 = as_half2(w & 0x00F000F0u);   // 1, 5 (x16)
            const half2_t w2 = as_half2(w8 & 0x000F000Fu);  // 2, 6
            const half2_t w3 = as_half2(w8 & 0x00F000F0u);  // 3, 7 (x16)
#pragma unroll
            for (int t = 0; t < NR; ++t) {
              p[t] = __builtin_amdgcn_fdot2(w0, as_half2(xv[t][i][0]), p[t], false);
              p[t] = __builtin_amdgcn_fdot2(w1, as_half2(xv[t][i][1]), p[t], false);
              p[t] = __builtin_amdgcn_fdot2(w2, as_half2(xv[t][i][2]), p[t], false);
              p[t] = __builtin_amdgcn_fdot2(w3, as_half2(xv[t][i][3]), p[t], false);
            }
          }
          // sum x*(q-8) = 2^24 * p - 8 * sum(x), times the group's scale
          const float s = (float)__builtin_bit_cast(_Float16, (uint16_t)f.sc[b][m]);
#pragma unroll
          for (int t = 0; t < NR; ++t) acc[b][m][t] = fmaf(s, fmaf(p[t], 16777216.f, -cx[t]), acc[b][m][t]);
        }
    };

    // Ping-pong over whole super-steps: the next one's loads are issued
    // before the current one is computed (a scheduling fence keeps them
    // there), so a wave always has one super-step in flight.  The loop runs
    // while two remain and the last one or two are peeled, so every load is
    // used and the load counters stay exact.
    {
      const int last = S_end_full - 1;
      int S = S_begin;
      for (; S + 2 <= last; S += 2) {
        load_super(S + 1, fb, true);
        __builtin_amdgcn_sched_barrier(0);
        compute_super(S, fa);
        load_super(S + 2, fa, true);
        __builtin_amdgcn_sched_barrier(0);
        compute_super(S + 1, fb);
      }
      if (S + 1 == last) {
        load_super(S + 1, fb, true);
        __builtin_amdgcn_sched_barrier(0);
        compute_super(S, fa);
        compute_super(S + 1, fb);
      } else if (S == last) {
        compute_super(S, fa);
      }
      if (has_tail) {  // the partial super-step: lanes past the last group read 0
        load_super(nss_full, fa, nss_full * 16 + j < ngroups);
        compute_super(nss_full, fa);
      }
    }

    // ---- add over the 16 lanes of a row (they hold different groups); then
    // lane (q, j < 4) takes row 4j + q of each block
    float res[NBB][NR];
#pragma unroll
    for (int b = 0; b < NBB; ++b)
#pragma unroll
      for (int t = 0; t < NR; ++t) {
#pragma unroll
        for (int m = 0; m < 4; ++m) {
          float v = acc[b][m][t];
          v += __shfl_xor(v, 1, 64);
          v += __shfl_xor(v, 2, 64);
          v += __shfl_xor(v, 4, 64);
          v += __shfl_xor(v, 8, 64);
          acc[b][m][t] = v;
        }
        res[b][t] = j == 0 ? acc[b][0][t] : j == 1 ? acc[b][1][t] : j == 2 ? acc[b][2][t] : acc[b][3][t];
      }
    const int r = 4 * j + q;  // this lane's row in each block (lanes with j < 4)
    // ---- split-K: every split stores its partial sums and takes a ticket;
    // the last to arrive reads all of them and adds them in split order, so
    // the sum does not depend on the order of arrival, then runs the epilogue.
    // No block waits.  (A device-scope release and acquire around the ticket
    // write back and invalidate the XCD's L2: measured 4x slower on MI355X.)
    if (g.splits > 1) {
      __shared__ int s_last;
      const int tile = item * g.nblk + nb;
      // partials go through with system-coherent stores (write-through past
      // the XCD's L2) and are read back with system-coherent loads, so no L2
      // writeback or invalidate is needed around the ticket
      const __amdgpu_buffer_rsrc_t rP = buffer_rsrc(g.part + (size_t)tile * g.splits * 256, (uint32_t)g.splits * 1024);
      constexpr int kSys = 1 | 16;  // sc0 | sc1
      if (j < 4) {
#pragma unroll
        for (int b = 0; b < NBB; ++b)
#pragma unroll
          for (int t = 0; t < NR; ++t)
            __builtin_amdgcn_raw_buffer_store_b32(__float_as_uint(res[b][t]), rP,
                                                  4 * (split * 256 + (wn * 4 + b * NR + t) * 16 + r), 0, kSys);
      }
      wait_vmcnt<0>();  // the partials have reached memory
      __syncthreads();
      if (tid == 0) s_last = atomicAdd(&g.tickets[tile], 1) == g.splits - 1;
      __syncthreads();
      if (!s_last) return;
      if (j < 4) {
#pragma unroll
        for (int b = 0; b < NBB; ++b)
#pragma unroll
          for (int t = 0; t < NR; ++t) {
            const uint32_t o = 4 * ((wn * 4 + b * NR + t) * 16 + r);
            float v = __uint_as_float(__builtin_amdgcn_raw_buffer_load_b32(rP, o, 0, kSys));
            for (int sp = 1; sp < g.splits; ++sp)
              v += __uint_as_float(__builtin_amdgcn_raw_buffer_load_b32(rP, o + sp * 1024, 0, kSys));
            res[b][t] = v;
          }
      }
      if (tid == 0) g.tickets[tile] = 0;
    }
    if (j >= 4) return;

    // ---- epilogue: lane (q, j) holds weight row r = 4j + q of each block
#pragma unroll
    for (int t = 0; t < NR; ++t) {
      if (t >= nr) continue;
      const int pos = pos0 + t;
      if (GATEUP) {
        if (col0[0] >= g.N) continue;
        const int col = col0[0] + r;
        // g = res * 2^e; h is stored times 2^-2e, odd columns divided by 16
        const float gt = res[0][t] * sc_of[t];
        const float up = res[1][t] * inv_pow2f(sc_of[t]) * ((col & 1) ? 0.0625f : 1.0f);
        g.h_out[(size_t)pos * g.N + ((col & ~7) | inv_perm8(col & 7))] = silu_mul_h(gt, up);
      } else {
        const int slot = slot_of[t];
        if (slot < 0 || slot >= g.R) continue;
        const float wv = sc_of[t];
#pragma unroll
        for (int c = 0; c < NBW; ++c) {
          if (col0[c] >= g.N) continue;
          g.y_out[(size_t)slot * g.N + col0[c] + r] = (uint16_t)f32_to_bf16_rne(wv * res[c][t]);
        }
      }
    }
  };
  if (nr == 1) path(std::integral_constant<int, 1>{});
  else path(std::integral_constant<int, 2>{});
}

// ---------------------------------------------------------------- combine

// out[t, n] = sum_{j<k} y[t*k + j, n] (in j order) + y[T + t, n] if shared,
// summed in fp32 from the bf16 slot rows and rounded to bf16.  One thread
// per 4 consecutive columns; the k slots are loaded in batches of 8 before
// they are summed, so a thread waits for one round trip per batch rather
// than one per slot.  SHARD: an expert-parallel shard, whose slots routed
// to experts outside [lo, lo + nloc) have no rows and are skipped.
template <bool SHARD>
__global__ __launch_bounds__(kThreads) void combine_kernel(const uint2* y, uint2* out, int M, int H, int k,
                                                            int T, int S, const int* ids, int lo, int nloc) {
  const long long q = (long long)blockIdx.x * kThreads + threadIdx.x;
  const int per_row = H / 4;
  if (q >= (long long)M * per_row) return;
  const int t = (int)(q / per_row), c4 = (int)(q % per_row);
  const uint2* base = y + (size_t)c4;
  const size_t row4 = (size_t)H / 4;
  float4 acc = make_float4(0.f, 0.f, 0.f, 0.f);
  const int n = k + (S ? 1 : 0);  // slot rows to add, the shared expert last
  for (int j0 = 0; j0 < n; j0 += 8) {
    uint2 v[8];
    bool use[8];
#pragma unroll
    for (int u = 0; u < 8; ++u) {
      const int j = j0 + u;
      use[u] = j < n;
      if (SHARD && j < k) {
        const int le = ids[(size_t)t * k + j] - lo;
        use[u] = le >= 0 && le < nloc;
      }
      const size_t r = j < k ? (size_t)t * k + j : (size_t)T + t;
      v[u] = use[u] ? base[r * row4] : make_uint2(0u, 0u);
    }
#pragma unroll
    for (int u = 0; u < 8; ++u) {
      if (use[u]) {
        acc.x += __uint_as_float(v[u].x << 16);
        acc.y += __uint_as_float(v[u].x & 0xFFFF0000u);
        acc.z += __uint_as_float(v[u].y << 16);
        acc.w += __uint_as_float(v[u].y & 0xFFFF0000u);
      }
    }
  }
  uint2 o;
  o.x = f32_to_bf16_rne(acc.x) | (f32_to_bf16_rne(acc.y) << 16);
  o.y = f32_to_bf16_rne(acc.z) | (f32_to_bf16_rne(acc.w) << 16);
  out[q] = o;
}

// ----------------------------------------------------------------- router

// The router in front of the layer: logits[t, e] = sum_k x[t, k] * W_r[e, k]
// with bf16 x [M, H] and bf16 W_r [E, H], accumulated in fp32 (products of
// two bf16 values are exact in fp32).  The pages state top-8 routing over
// 384 experts but not the router ("The MoE Throughput Lever: Quantifying the
// INT4 Marlin GEMM on Blackwell PRO 6000", section "The Context: Why This
// Measurement Matters"): a linear map to one logit per expert is the
// plainest reading.

struct RouterArgs {
  const uint4* x;   // bf16 [M, H] as 16-byte runs
  const uint4* wr;  // bf16 [E, H]
  float* logits;    // fp32 [M, E]
  int M, E, H;
};

constexpr int kRouterGemvTokens = 4;   // tokens per wave of the GEMV
constexpr int kRouterGemvMaxM = 16;    // the GEMV up to this many tokens, tiles above

// bf16 pair (one dword) dotted with another, accumulated by two fp32 FMAs
__device__ __forceinline__ float dot_bf16x2(uint32_t a, uint32_t b, float acc) {
  acc = fmaf(bf16_lo(a), bf16_lo(b), acc);
  return fmaf(bf16_hi(a), bf16_hi(b), acc);
}

// Small M: one wave per (expert, group of up to 4 tokens); each lane takes
// 8 consecutive inputs of every 512, the 64 lanes' partial sums are added by
// a butterfly.  The router row is read once per token group, x from cache.
// The loads of kRouterGemvSteps loop steps go out before their products, so
// a 7168-input row is 4 round trips to memory rather than 14 (each lane
// still adds its products in input order).
constexpr int kRouterGemvSteps = 4;
__global__ __launch_bounds__(kThreads) void router_gemv_kernel(RouterArgs a) {
  const int lane = threadIdx.x & 63;
  const int wid = (int)blockIdx.x * (kThreads / 64) + (int)(threadIdx.x >> 6);
  const int e = wid % a.E, tg = wid / a.E;
  const int t0 = tg * kRouterGemvTokens;
  if (t0 >= a.M) return;
  const int runs = a.H / 8;
  const uint4* wrow = a.wr + (size_t)e * runs;
  const uint4* xrow[kRouterGemvTokens];
#pragma unroll
  for (int u = 0; u < kRouterGemvTokens; ++u) xrow[u] = a.x + (size_t)min(t0 + u, a.M - 1) * runs;  // clamped
  float acc[kRouterGemvTokens] = {};
  int v = lane;
  for (; v + (kRouterGemvSteps - 1) * 64 < runs; v += kRouterGemvSteps * 64) {
    uint4 w[kRouterGemvSteps], xv[kRouterGemvSteps][kRouterGemvTokens];
#pragma unroll
    for (int s = 0; s < kRouterGemvSteps; ++s) {
      w[s] = wrow[v + 64 * s];
#pragma unroll
      for (int u = 0; u < kRouterGemvTokens; ++u) xv[s][u] = xrow[u][v + 64 * s];
    }
#pragma unroll
    for (int s = 0; s < kRouterGemvSteps; ++s)
#pragma unroll
      for (int u = 0; u < kRouterGemvTokens; ++u) {
        acc[u] = dot_bf16x2(w[s].x, xv[s][u].x, acc[u]);
        acc[u] = dot_bf16x2(w[s].y, xv[s][u].y, acc[u]);
        acc[u] = dot_bf16x2(w[s].z, xv[s][u].z, acc[u]);
        acc[u] = dot_bf16x2(w[s].w, xv[s][u].w, acc[u]);
      }
  }
  for (; v < runs; v += 64) {
    const uint4 w = wrow[v];
#pragma unroll
    for (int u = 0; u < kRouterGemvTokens; ++u) {
      const uint4 xv = xrow[u][v];
      acc[u] = dot_bf16x2(w.x, xv.x, acc[u]);
      acc[u] = dot_bf16x2(w.y, xv.y, acc[u]);
      acc[u] = dot_bf16x2(w.z, xv.z, acc[u]);
      acc[u] = dot_bf16x2(w.w, xv.w, acc[u]);
    }
  }
#pragma unroll
  for (int u = 0; u < kRouterGemvTokens; ++u) {
    float v = acc[u];
#pragma unroll
    for (int m = 32; m >= 1; m >>= 1) v += __shfl_xor(v, m, 64);
    if (lane == 0 && t0 + u < a.M) a.logits[(size_t)(t0 + u) * a.E + e] = v;
  }
}

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
constexpr int kRouterTok = 32;      // tokens per block (two halves of 16)
constexpr int kRouterExp = 64;      // experts per block
constexpr int kRouterKC = 64;       // inputs per K chunk (two MFMA k-slices)
constexpr int kRouterKSplit = 8;    // K chunks dealt round-robin to 8 wave pairs
constexpr int kRouterThreads = 64 * 2 * kRouterKSplit;

// Larger M: 32-token x 64-expert tiles; bf16 MFMA 16x16x32 with fp32
// accumulators.  The block's 16 waves are 2 token halves x 8 K groups: group
// g takes K chunks g, g + 8, g + 16, ..., so each wave's chain of dependent
// chunk loads is an eighth of K long (a 7168-input row in 14 chunk steps
// rather than 112).  The router's whole input is a few MB, so the call is
// bound by that chain, not by bytes: on MI355X (384 experts, 7168 inputs)
// 90 and 1024 tokens took about 34 us against 90 us with one K group (four
// groups: 39 us); at 4096 tokens it stays near 92 us, set by the chain
// times the rounds of blocks (one per CU at 128 KiB of LDS).
// Each group's chunk of the router rows (64 rows x 128 bytes) goes from
// memory straight into the group's LDS buffer (lane l of a load instruction
// fills bytes 16l..16l+15 of its 1 KiB), double-buffered; the 16-byte piece
// p of row n sits at slot p ^ ((n >> 1) & 7), so the 16 rows an MFMA operand
// read touches fall in distinct banks.  Each wave's token fragments come
// from memory into registers, one chunk ahead.  All waves run the same
// number of steps (a group past the last chunk loads and adds zeros), and
// the groups' partial tiles are added through LDS in group order.
__global__ __launch_bounds__(kRouterThreads) void router_tile_kernel(RouterArgs a) {
  __shared__ __attribute__((aligned(16))) _Float16 lds_w[kRouterKSplit * 2 * kRouterExp * kRouterKC];
  static_assert(sizeof(lds_w) >= kRouterThreads * 16 * sizeof(float), "the partial tiles fit the buffers");
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int th = wave & 1, kg = wave >> 1;  // token half, K group
  const int r = lane & 15, kq = lane >> 4;
  const int ntt = (a.M + kRouterTok - 1) / kRouterTok;
  const int t0 = ((int)blockIdx.x % ntt) * kRouterTok, e0 = ((int)blockIdx.x / ntt) * kRouterExp;
  const uint32_t row_bytes = (uint32_t)a.H * 2;
  const __amdgpu_buffer_rsrc_t rX = buffer_rsrc(a.x, (uint32_t)a.M * row_bytes);
  const __amdgpu_buffer_rsrc_t rW = buffer_rsrc(a.wr, (uint32_t)a.E * row_bytes);
  // this lane's token row (rows past M read zeros)
  const int trow = t0 + 16 * th + r;
  const uint32_t xoff = trow < a.M ? (uint32_t)trow * row_bytes + 16 * kq : kOob;
  // router-row loads: the group's two waves fill its 64 rows, instruction j
  // of wave th rows 8(4th + j) .. +7; lane l: row + l/8, slot l%8
  uint32_t woff[4];
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    const int n = 8 * (4 * th + j) + (lane >> 3);
    const int piece = (lane & 7) ^ ((n >> 1) & 7);
    woff[j] = e0 + n < a.E ? (uint32_t)(e0 + n) * row_bytes + 16 * piece : kOob;
  }
  _Float16* const gw = lds_w + kg * 2 * kRouterExp * kRouterKC;  // this group's two buffers
  const int nchunks = a.H / kRouterKC;
  const int steps = (nchunks + kRouterKSplit - 1) / kRouterKSplit;
  // chunk of step it for this group; past the last one every lane reads zeros
  auto load_w = [&](int it, int buf) __attribute__((always_inline)) {
    const int c = kRouterKSplit * it + kg;
#pragma unroll
    for (int j = 0; j < 4; ++j)
      load_lds16(rW, gw + buf * kRouterExp * kRouterKC + (8 * (4 * th + j)) * kRouterKC, c < nchunks ? woff[j] : kOob,
                 c * kRouterKC * 2);
  };
  auto load_x = [&](int it, u32x4_t (&xf)[2]) __attribute__((always_inline)) {
    const int c = kRouterKSplit * it + kg;
#pragma unroll
    for (int s = 0; s < 2; ++s)
      xf[s] = __builtin_bit_cast(
          u32x4_t, __builtin_amdgcn_raw_buffer_load_b128(rX, c < nchunks ? xoff : kOob, c * kRouterKC * 2 + 64 * s, 0));
  };
  float4_t acc[4];
#pragma unroll
  for (int cb = 0; cb < 4; ++cb) acc[cb] = float4_t{0.f, 0.f, 0.f, 0.f};
  u32x4_t xa[2], xb[2];
  load_w(0, 0);
  load_x(0, xa);
  wait_vmcnt<0>();
  __syncthreads();
  for (int it = 0; it < steps; ++it) {
    const int buf = it & 1;
    const bool more = it + 1 < steps;
    if (more) {
      load_w(it + 1, buf ^ 1);
      load_x(it + 1, xb);
    }
    __builtin_amdgcn_sched_barrier(0);
    const _Float16* lb = gw + buf * kRouterExp * kRouterKC;
#pragma unroll
    for (int s = 0; s < 2; ++s) {
      const bf16x8_t av = __builtin_bit_cast(bf16x8_t, xa[s]);
#pragma unroll
      for (int cb = 0; cb < 4; ++cb) {
        const int n = 16 * cb + r, piece = 4 * s + kq;
        const u32x4_t bv = *reinterpret_cast<const u32x4_t*>(lb + n * kRouterKC + 8 * (piece ^ ((n >> 1) & 7)));
        acc[cb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(av, __builtin_bit_cast(bf16x8_t, bv), acc[cb], 0, 0, 0);
      }
    }
    wait_vmcnt<0>();
    __syncthreads();
    xa[0] = xb[0];
    xa[1] = xb[1];
  }
  // the groups' partial tiles through LDS (the loop ended on a barrier, so
  // the buffers are free), added in group order by the waves of group 0
  float* red = reinterpret_cast<float*>(lds_w);
#pragma unroll
  for (int cb = 0; cb < 4; ++cb)
#pragma unroll
    for (int i = 0; i < 4; ++i) red[((wave * 4 + cb) * 4 + i) * 64 + lane] = acc[cb][i];
  __syncthreads();
  if (kg != 0) return;
  // lane (r, kq) holds tokens 4kq..4kq+3 of its half's 16, expert column r
#pragma unroll
  for (int cb = 0; cb < 4; ++cb) {
    const int e = e0 + 16 * cb + r;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      float v = red[((th * 4 + cb) * 4 + i) * 64 + lane];
#pragma unroll
      for (int g = 1; g < kRouterKSplit; ++g) v += red[(((th + 2 * g) * 4 + cb) * 4 + i) * 64 + lane];
      const int t = t0 + 16 * th + 4 * kq + i;
      if (t < a.M && e < a.E) a.logits[(size_t)t * a.E + e] = v;
    }
  }
}


// ------------------------------------------------------- code tile order

// The layer's copy of a code array in tile order (tiled_code_offset): one
// thread per 16-byte chunk of the destination, so the writes are whole
// lines; rows is a multiple of 16 and K2 = K/2 of 64.
__global__ __launch_bounds__(kThreads) void tile_codes_kernel(const uint4* __restrict__ src, uint4* __restrict__ dst,
                                                               long long chunks, int K2) {
  const long long c = (long long)blockIdx.x * kThreads + threadIdx.x;
  if (c >= chunks) return;
  const long long blk = c / K2;  // 16-row block: 16 * K2 bytes = K2 chunks
  const int w = (int)(c % K2), sub = w / 64, l = w % 64;
  const long long n = blk * 16 + (l & 15);  // row r = l % 16, lane part kq = l / 16
  dst[c] = src[(n * K2 + sub * 64 + (l >> 4) * 16) / 16];
}

// The same for a scale array (tiled_scale_offset): one thread per 8-byte
// chunk of the destination (four groups of one row); KG = K/32 is a
// multiple of 4.
__global__ __launch_bounds__(kThreads) void tile_scales_kernel(const uint2* __restrict__ src, uint2* __restrict__ dst,
                                                                long long chunks, int KG) {
  const long long c = (long long)blockIdx.x * kThreads + threadIdx.x;
  if (c >= chunks) return;
  const long long blk = c / (4 * KG);  // 16-row block: 16 * KG * 2 bytes = 4 KG chunks
  const int w = (int)(c % (4 * KG)), S = w / 64, l = w % 64;
  const long long n = blk * 16 + (l & 15);  // row r = l % 16, group quad kq = l / 16
  dst[c] = src[(n * KG + S * 16 + (l >> 4) * 4) / 4];
}

// ------------------------------------------------------------- inspection

// w, s: one expert's codes and scales in tile order (K2 = K/2 bytes per row)
__global__ __launch_bounds__(kThreads) void dequant_kernel(const uint32_t* w, const uint16_t* s, int N,
                                                            int K, uint16_t* out) {
  const long long idx = (long long)blockIdx.x * kThreads + threadIdx.x;
  const int per_row = K / 8;
  if (idx >= (long long)N * per_row) return;
  const int n = (int)(idx / per_row), d = (int)(idx % per_row);
  half8_t v = dq8(w[tiled_code_offset(n, 4 * (size_t)d, K / 2) / 4], s[tiled_scale_offset(n, d / 4, K / 32) / 2]);
#pragma unroll
  for (int p = 0; p < 8; ++p)
    if (x16_pos(p)) v[p] = v[p] * (_Float16)0.0625f;  // exact: undo the operand's x16
  // bit-cast the whole vector (a bit-cast of one vector element reads element 0)
  const u16x8_t h = __builtin_bit_cast(u16x8_t, v);
#pragma unroll
  for (int p = 0; p < 8; ++p) out[(size_t)n * K + d * 8 + perm8(p)] = h[p];
}

// h rows are held in sorted order, times 2^-2e of their token, odd columns
// divided by 16; out: slot order, true scale.
__global__ __launch_bounds__(kThreads) void read_h_kernel(const _Float16* h, const int* inv_perm,
                                                           const int* xexp, int T, int k, long long R, int I,
                                                           float* out) {
  const long long q = (long long)blockIdx.x * kThreads + threadIdx.x;
  if (q >= R * I) return;
  const long long f = q / I;
  const int col = (int)(q % I);
  long long pos = f < T ? inv_perm[f] : f;
  if (pos < 0 || pos >= R) pos = f;
  const long long tok = f < T ? f / k : f - T;
  const float v = (float)h[pos * I + ((col & ~7) | inv_perm8(col & 7))] * pow2f(2 * xexp[tok]);
  out[q] = (col & 1) ? v * 16.0f : v;
}

__global__ __launch_bounds__(kThreads) void read_y_kernel(const uint16_t* y, long long n, float* out) {
  const long long q = (long long)blockIdx.x * kThreads + threadIdx.x;
  if (q < n) out[q] = __uint_as_float((uint32_t)y[q] << 16);
}

__global__ void init_ctrl_kernel(int* ctrl) {
  if (threadIdx.x < kCtrlWords) ctrl[threadIdx.x] = 0;
}

// ============================================================= host side

thread_local std::string g_err;
// receipt of the forward call being enqueued on this thread (null outside one)
thread_local qmoe_receipt* t_rc = nullptr;

int fail(int code, const std::string& msg) {
  g_err = msg;
  return code;
}

size_t align256(size_t v) { return (v + 255) & ~(size_t)255; }

struct Layout {
  int64_t T, S, R, C, max_items_all;
  size_t ctrl, ids, wts, counts, offsets, perm, inv_perm, items, items_gv, xexp, logits, xa, h, y, part, tickets,
      total;
  int splits_gu, splits_dn;  // GEMV split-K of the call (1 = none)
  int64_t n_tickets;
};

int64_t ceil_div(int64_t a, int64_t b) { return (a + b - 1) / b; }

int64_t max_items_for(int64_t T, int64_t M, int64_t S, int64_t E, int64_t bmc) {
  return T / bmc + std::min<int64_t>(E, T) + (S ? ceil_div(M, bmc) : 0);
}

}  // namespace

// Scratch of qmoe_forward_static (callers that cannot allocate device
// memory): one file-scope device array per GPU, used in place of a caller
// workspace.  In host code `scratch` names a host-side stand-in; its device
// address on each GPU comes from hipGetSymbolAddress, taken once per device
// when the first layer on that device is created, and only that address is
// ever passed to kernels.
namespace {
constexpr size_t kScratchBytes = (size_t)QMOE_STATIC_SCRATCH_BYTES;
constexpr int kMaxDevices = 64;
static __device__ __align__(256) uint8_t scratch[kScratchBytes];
std::mutex g_scratch_mu;
void* g_scratch_ptr[kMaxDevices] = {};

// The device address of `scratch` on device dev (the current device).
hipError_t scratch_address(int dev, void** out) {
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
  if (g_scratch_ptr[dev] == nullptr) {
    void* p = nullptr;
    const hipError_t e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess) return e;
    g_scratch_ptr[dev] = p;
  }
  *out = g_scratch_ptr[dev];
  return hipSuccess;
}
}  // namespace

struct qmoe_layer {
  qmoe_layer_desc d;
  int device = 0;
  bool shared = false;
  int lo = 0, nloc = 0;     // local experts [lo, lo + nloc) (all E unless a shard)
  float rscale = 1.0f;      // routed scaling factor of the sigmoid scoring
  void* scratch = nullptr;  // device address of this device's scratch array
  std::mutex receipt_mu;
  qmoe_receipt last{};      // receipt of the last completed forward call
  bool has_receipt = false;
  std::atomic<uint64_t> receipt_seq{0};  // forward calls since creation (not reset by qmoe_reset_stats)
  std::atomic<uint64_t> forward_calls{0}, route_calls{0}, gemm_launches{0}, launches{0}, inits{0},
      ws_last{0}, ws_peak{0}, prefill_tiles{0}, gemv_tiles{0}, gemv_nt{0}, splitk_launches{0};
  // the codes and scales in tile order: one device allocation made at
  // creation and freed at destruction (the descriptor's pointers to them are
  // read once)
  void* tiled = nullptr;
  const uint8_t *w13 = nullptr, *w2 = nullptr, *sh_w13 = nullptr, *sh_w2 = nullptr;
  const uint16_t *s13 = nullptr, *s2 = nullptr, *sh_s13 = nullptr, *sh_s2 = nullptr;
};

namespace {

enum Regime { kGemv, kPrefill };
Regime regime_of(const qmoe_layer* L, int64_t M);
int gemv_splits(const qmoe_layer* L, int64_t M, bool gateup, int64_t* tiles);

Layout make_layout(const qmoe_layer* L, int64_t M) {
  Layout l{};
  const int64_t E = L->d.E, H = L->d.H, I = L->d.I, k = L->d.top_k;
  l.T = M * k;
  l.S = L->shared ? M : 0;
  l.R = l.T + l.S;
  l.C = ceil_div(M, kChunk);
  l.max_items_all = max_items_for(l.T, M, l.S, L->nloc, kGemvRows);  // the smallest row tile bounds all
  size_t off = 0;
  auto take = [&](size_t bytes) {
    const size_t o = off;
    off = align256(off + bytes);
    return o;
  };
  l.ctrl = take(kCtrlWords * 4);
  l.ids = take(l.T * 4);
  l.wts = take(l.T * 4);
  l.counts = take((L->nloc + 1) * 4);
  l.offsets = take((L->nloc + 2) * 4);
  l.perm = take(l.R * 4);
  l.inv_perm = take(l.T * 4);
  l.items = take(l.max_items_all * 16);
  l.items_gv = take(L->nloc * 16);
  l.xexp = take(M * 4);
  l.logits = take(M * E * 4);  // router logits of qmoe_forward_router
  l.xa = take(M * H * 2);
  l.h = take(l.R * I * 2);
  l.y = take(l.R * H * 2);
  // GEMV split-K partial sums and tickets (small calls only)
  l.splits_gu = l.splits_dn = 1;
  l.n_tickets = 0;
  if (M > 0 && regime_of(L, M) == kGemv) {
    int64_t tg = 0, td = 0;
    l.splits_gu = gemv_splits(L, M, true, &tg);
    l.splits_dn = gemv_splits(L, M, false, &td);
    const int64_t pg = l.splits_gu > 1 ? tg * l.splits_gu : 0, pd = l.splits_dn > 1 ? td * l.splits_dn : 0;
    if (pg || pd) l.n_tickets = std::max(l.splits_gu > 1 ? tg : 0, l.splits_dn > 1 ? td : 0);
    l.part = take(std::max(pg, pd) * 256 * 4);
  } else {
    l.part = take(0);
  }
  l.tickets = take(l.n_tickets * 4);
  l.total = off;
  return l;
}

// Kernel regime of a call, from the average routed rows per expert: the
// dot-product GEMV (items of <= 2 rows) up to 1.75 rows on average, 128-row
// MFMA tiles above.  An expert with more than 2 rows takes several GEMV
// items, each streaming its weights.  Measured on MI355X (E=384, H=7168,
// I=2048, top-8): the GEMV is ahead at 1.33 rows per expert (M=64, 7%),
// the tiles at 2 (M=96, 3%) and 4 (M=192, 30%).  The GEMV stages two
// activation rows in LDS, so it is used while they fit in 64 KiB.
static_assert(gemv_lds_bytes(kGemvMaxK) <= 65536, "GEMV rows fit in 64 KiB of LDS");
Regime regime_of(const qmoe_layer* L, int64_t M) {
  const int64_t T = M * (int64_t)L->d.top_k, E = L->d.E;
  if (4 * T <= kGemvMaxRowsPer4Experts * E && L->d.H <= kGemvMaxK && L->d.I <= kGemvMaxK) return kGemv;
  return kPrefill;
}
int rows_per_item(Regime rg) { return rg == kGemv ? kGemvRows : kPrefillRows; }

// A mixed call: in the tile regime, while calls average at most
// kMixedMaxRowsPerExpert routed rows per expert, a routed expert of 1 or 2
// rows takes one dot-product GEMV item (a second work list) instead of a
// 128-row tile item: the GEMV streams an expert's weights faster per block
// than a tile does, and such an expert's tile computes mostly zero rows.
// Each product then runs the tile launch and a GEMV launch over that list.
// Measured on MI355X (E=384, H=7168, I=2048, top-8): at M=90 (1.9 rows per
// expert, two thirds of the touched experts light) the call 1,700 -> 1,539
// us; at 256 tokens (5.3 rows, a tenth light) and on the skewed 512-token
// call within 1%, while the I=256 and 48-expert slices at 256 tokens ran
// 5-7% slower (the extra launches outweigh their few light experts).
constexpr int kMixedMaxRowsPerExpert = 4;
bool mixed_call(const qmoe_layer* L, int64_t M) {
  return regime_of(L, M) == kPrefill && M * L->d.top_k <= kMixedMaxRowsPerExpert * (int64_t)L->d.E &&
         L->d.H <= kGemvMaxK && L->d.I <= kGemvMaxK;
}

// Split-K of a GEMV launch: a grid of fewer than kSplitMaxTiles blocks (a
// few experts with narrow rows: one GPU's share of a tensor-parallel layer
// at decode sizes) is split along K, into up to one split per whole
// super-step and about kSplitTargetBlocks blocks in all, so that the stream
// runs on more CUs.  Measured on MI355X: the 384-expert I=256 slice at one
// token, gate+up 22.4 -> 21.0 us with 11 splits; the whole layer at one
// token (384 tiles), 29.4 -> 30.9 us with 2 splits, so larger grids stay
// whole.  *tiles: blocks of the unsplit grid (item x column block).
constexpr int kSplitMaxTiles = 128;
constexpr int kSplitTargetBlocks = 512;
int gemv_splits(const qmoe_layer* L, int64_t M, bool gateup, int64_t* tiles) {
  const int64_t T = M * L->d.top_k, S = L->shared ? M : 0;
  const int64_t max_items = max_items_for(T, M, S, L->nloc, kGemvRows);
  const int64_t N = gateup ? L->d.I : L->d.H;
  const int64_t nblk = ceil_div(N, (kThreads / 64) * (gateup ? 16 : 32));
  *tiles = max_items * nblk;
  const int64_t nss_full = (gateup ? L->d.H : L->d.I) / kSuper;
  if (*tiles >= kSplitMaxTiles || nss_full < 2) return 1;
  return (int)std::min<int64_t>(nss_full, ceil_div(kSplitTargetBlocks, *tiles));
}

template <typename T>
T* at(void* ws, size_t off) {
  return reinterpret_cast<T*>(static_cast<char*>(ws) + off);
}

int check_launch(qmoe_layer* L, const char* what) {
  L->launches++;
  if (t_rc) t_rc->launches++;
  const hipError_t e = hipGetLastError();
  if (e != hipSuccess) return fail(QMOE_ERR_LAUNCH, std::string(what) + ": " + hipGetErrorString(e));
  return QMOE_OK;
}

int check_call(qmoe_layer* L, int64_t M, const void* ws, size_t ws_bytes, Layout* lay) {
  if (!L) return fail(QMOE_ERR_ARG, "layer is NULL");
  if (M < 0 || M > L->d.max_rows)
    return fail(QMOE_ERR_ARG, "M=" + std::to_string(M) + " outside [0, max_rows=" +
                                  std::to_string(L->d.max_rows) + "]");
  *lay = make_layout(L, M);
  if (M == 0) return QMOE_OK;
  if (!ws) return fail(QMOE_ERR_WORKSPACE, "workspace is NULL");
  if ((reinterpret_cast<uintptr_t>(ws) & 255) != 0) return fail(QMOE_ERR_WORKSPACE, "workspace not 256-byte aligned");
  if (ws_bytes < lay->total)
    return fail(QMOE_ERR_WORKSPACE, "workspace has " + std::to_string(ws_bytes) + " bytes, M=" +
                                        std::to_string(M) + " needs " + std::to_string(lay->total));
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess) return fail(QMOE_ERR_DEVICE, "hipGetDevice failed");
  if (dev != L->device)
    return fail(QMOE_ERR_DEVICE, "current device " + std::to_string(dev) + " is not the layer's device " +
                                     std::to_string(L->device));
  L->ws_last = lay->total;
  uint64_t peak = L->ws_peak.load();
  while (lay->total > peak && !L->ws_peak.compare_exchange_weak(peak, lay->total)) {
  }
  return QMOE_OK;
}

int init_workspace(qmoe_layer* L, void* ws, size_t ws_bytes, hipStream_t st) {
  (void)ws_bytes;
  init_ctrl_kernel<<<1, kCtrlWords, 0, st>>>(static_cast<int*>(ws));
  L->inits++;
  return check_launch(L, "workspace init");
}

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15) == 0; }

int do_route(qmoe_layer* L, const void* x, const float* logits, int64_t M, void* ws, const Layout& lay,
             hipStream_t st) {
  if (!x || !logits) return fail(QMOE_ERR_ARG, x ? "logits is NULL" : "x is NULL");
  if (!aligned16(x)) return fail(QMOE_ERR_ARG, "x must be 16-byte aligned");
  const int bmc = rows_per_item(regime_of(L, M));
  RouteArgs a;
  a.logits = logits;
  a.x = static_cast<const uint4*>(x);
  a.M = (int)M;
  a.E = L->d.E;
  a.H = L->d.H;
  a.k = L->d.top_k;
  a.S = (int)lay.S;
  a.C = (int)lay.C;
  a.bmc = bmc;
  a.max_items = (int)max_items_for(lay.T, M, lay.S, L->nloc, bmc);
  a.lo = L->lo;
  a.nloc = L->nloc;
  a.scoring = L->d.scoring;
  a.rscale = L->rscale;
  a.bias = L->d.expert_bias;
  a.ctrl = at<int>(ws, lay.ctrl);
  a.ids = at<int>(ws, lay.ids);
  a.wts = at<float>(ws, lay.wts);
  a.counts = at<int>(ws, lay.counts);
  a.offsets = at<int>(ws, lay.offsets);
  a.perm = at<int>(ws, lay.perm);
  a.inv_perm = at<int>(ws, lay.inv_perm);
  a.items = at<int4>(ws, lay.items);
  a.items_gv = at<int4>(ws, lay.items_gv);
  a.gv = mixed_call(L, M) ? kGemvRows : 0;
  a.xa = at<uint4>(ws, lay.xa);
  a.xexp = at<int>(ws, lay.xexp);
  a.tickets = at<int>(ws, lay.tickets);
  a.n_tickets = (int)lay.n_tickets;
  const int epl = (L->d.E + 63) / 64;
  L->route_calls++;
  if (lay.C == 1) {
    // one routing block of one wave per token, then x-conversion blocks
    // of as many waves
    const int nw = (int)std::min<int64_t>(M, kRouteWaves);
    a.nrb = 1;
    const dim3 grid((unsigned)(1 + ceil_div(M, nw))), block((unsigned)(64 * nw));
    if (epl <= 1) route_single_kernel<1><<<grid, block, 0, st>>>(a);
    else if (epl <= 2) route_single_kernel<2><<<grid, block, 0, st>>>(a);
    else if (epl <= 4) route_single_kernel<4><<<grid, block, 0, st>>>(a);
    else if (epl <= 6) route_single_kernel<6><<<grid, block, 0, st>>>(a);  // 257-384 experts
    else if (epl <= 8) route_single_kernel<8><<<grid, block, 0, st>>>(a);
    else route_single_kernel<16><<<grid, block, 0, st>>>(a);
    return check_launch(L, "route_single_kernel");
  }
  // top-k blocks of 16 tokens, then as many x-conversion blocks; then one
  // finishing block per 64-token chunk
  a.nrb = (int)ceil_div(M, kRouteWaves);
  const dim3 grid((unsigned)(2 * a.nrb));
  if (epl <= 1) route_topk_kernel<1><<<grid, kRouteThreads, 0, st>>>(a);
  else if (epl <= 2) route_topk_kernel<2><<<grid, kRouteThreads, 0, st>>>(a);
  else if (epl <= 4) route_topk_kernel<4><<<grid, kRouteThreads, 0, st>>>(a);
  else if (epl <= 6) route_topk_kernel<6><<<grid, kRouteThreads, 0, st>>>(a);
  else if (epl <= 8) route_topk_kernel<8><<<grid, kRouteThreads, 0, st>>>(a);
  else route_topk_kernel<16><<<grid, kRouteThreads, 0, st>>>(a);
  int rc = check_launch(L, "route_topk_kernel");
  if (rc != QMOE_OK) return rc;
  route_finish_kernel<<<dim3((unsigned)lay.C), kRouteThreads, 0, st>>>(a);
  return check_launch(L, "route_finish_kernel");
}

template <bool GATEUP>
void fill_gemm_args(const qmoe_layer* L, int64_t M, void* ws, const Layout& lay, GemmArgs& g) {
  const int H = L->d.H, I = L->d.I;
  g.E = L->nloc;  // the weights hold the local experts
  g.T = (int)lay.T;
  g.M = (int)M;
  g.R = (int)lay.R;
  g.k = L->d.top_k;
  g.ctrl = at<int>(ws, lay.ctrl);
  g.count_at = 1;
  g.items = at<int4>(ws, lay.items);
  g.perm = at<int>(ws, lay.perm);
  g.wts = at<float>(ws, lay.wts);
  g.xexp = at<int>(ws, lay.xexp);
  g.splits = 1;
  g.part = at<float>(ws, lay.part);
  g.tickets = at<int>(ws, lay.tickets);
  if (GATEUP) {
    g.w = L->w13;
    g.s = L->s13;
    g.w_sh = L->sh_w13;
    g.s_sh = L->sh_s13;
    g.K = H;
    g.N = I;
    g.Nw = 2 * I;
    g.a = at<_Float16>(ws, lay.xa);
    g.a_bytes = (uint32_t)(M * H * 2);
    g.h_out = at<_Float16>(ws, lay.h);
    g.y_out = nullptr;
  } else {
    g.w = L->w2;
    g.s = L->s2;
    g.w_sh = L->sh_w2;
    g.s_sh = L->sh_s2;
    g.K = I;
    g.N = H;
    g.Nw = H;
    g.a = at<_Float16>(ws, lay.h);
    g.a_bytes = (uint32_t)(lay.R * I * 2);
    g.h_out = nullptr;
    g.y_out = at<uint16_t>(ws, lay.y);
  }
}

template <int MB, int WN, int NBW, bool GATEUP>
int launch_gemm(qmoe_layer* L, int64_t M, void* ws, const Layout& lay, hipStream_t st) {
  GemmArgs g;
  fill_gemm_args<GATEUP>(L, M, ws, lay, g);
  const int bmc = MB * 16;
  g.max_items = (int)max_items_for(lay.T, M, lay.S, L->nloc, bmc);
  g.nblk = (int)ceil_div(g.N, WN * NBW * 16);
  const int64_t blocks = 8 * (int64_t)g.nblk * ceil_div(g.max_items, 8);
  if (blocks > 0x7FFFFFFF) return fail(QMOE_ERR_UNSUPPORTED, "grid too large");
  gemm_kernel<MB, WN, NBW, GATEUP><<<dim3((unsigned)blocks), 64 * WN, 0, st>>>(g);
  L->gemm_launches++;
  if (t_rc) {
    t_rc->max_items = g.max_items;
    (GATEUP ? t_rc->gate_up_blocks : t_rc->down_blocks) = blocks;
  }
  return check_launch(L, GATEUP ? "gate_up gemm" : "down gemm");
}

template <bool GATEUP>
int launch_gemv(qmoe_layer* L, int64_t M, void* ws, const Layout& lay, hipStream_t st, bool mixed = false) {
  constexpr int WN = kThreads / 64;
  GemmArgs g;
  fill_gemm_args<GATEUP>(L, M, ws, lay, g);
  // the dot-product GEMV reads the codes as given (row order)
  g.w = GATEUP ? L->d.w13 : L->d.w2;
  g.w_sh = GATEUP ? L->d.shared_w13 : L->d.shared_w2;
  g.s = GATEUP ? L->d.s13 : L->d.s2;
  g.s_sh = GATEUP ? L->d.shared_s13 : L->d.shared_s2;
  if (mixed) {  // the light experts' list of a mixed call: at most one item per local expert
    g.items = at<int4>(ws, lay.items_gv);
    g.count_at = 2;
    g.max_items = L->nloc;
    g.splits = 1;
  } else {
    g.max_items = (int)max_items_for(lay.T, M, lay.S, L->nloc, kGemvRows);
    g.splits = GATEUP ? lay.splits_gu : lay.splits_dn;
  }
  const int cols = GATEUP ? 16 : 32;  // output columns per wave
  g.nblk = (int)ceil_div(g.N, WN * cols);
  const int64_t blocks = (int64_t)g.nblk * g.max_items * g.splits;
  if (blocks > 0x7FFFFFFF) return fail(QMOE_ERR_UNSUPPORTED, "grid too large");
  const size_t lds = gemv_lds_bytes(g.K);
  // non-temporal code reads while each expert's codes are read about once:
  // at most one routed row per expert on average and no shared expert (whose
  // codes every item of the call reads)
  const bool nt = !mixed && M * L->d.top_k <= L->d.E && L->d.shared_w13 == nullptr;
  if (nt) {
    gemv_kernel<GATEUP, true><<<dim3((unsigned)blocks), kThreads, lds, st>>>(g);
    L->gemv_nt++;
  } else
    gemv_kernel<GATEUP, false><<<dim3((unsigned)blocks), kThreads, lds, st>>>(g);
  L->gemm_launches++;
  if (g.splits > 1) L->splitk_launches++;
  if (t_rc && !mixed) {
    t_rc->max_items = g.max_items;
    t_rc->nt_codes = nt ? 1 : 0;
    (GATEUP ? t_rc->splits_gate_up : t_rc->splits_down) = g.splits;
    (GATEUP ? t_rc->gate_up_blocks : t_rc->down_blocks) = blocks;
  }
  return check_launch(L, GATEUP ? "gate_up gemv" : "down gemv");
}

int do_gate_up(qmoe_layer* L, int64_t M, void* ws, const Layout& lay, hipStream_t st) {
  if (regime_of(L, M) == kGemv) {
    L->gemv_tiles++;
    return launch_gemv<true>(L, M, ws, lay, st);
  }
  L->prefill_tiles++;
  const int rc = launch_gemm<kTileMB, kGuWN, kGuNBW, true>(L, M, ws, lay, st);
  if (rc != QMOE_OK || !mixed_call(L, M)) return rc;
  L->gemv_tiles++;
  return launch_gemv<true>(L, M, ws, lay, st, true);
}

int do_down(qmoe_layer* L, int64_t M, void* ws, const Layout& lay, hipStream_t st) {
  if (regime_of(L, M) == kGemv) return launch_gemv<false>(L, M, ws, lay, st);
  const int rc = launch_gemm<kTileMB, kDnWN, kDnNBW, false>(L, M, ws, lay, st);
  if (rc != QMOE_OK || !mixed_call(L, M)) return rc;
  return launch_gemv<false>(L, M, ws, lay, st, true);
}

int do_combine(qmoe_layer* L, int64_t M, void* out, void* ws, const Layout& lay, hipStream_t st) {
  if (!out) return fail(QMOE_ERR_ARG, "out is NULL");
  if (!aligned16(out)) return fail(QMOE_ERR_ARG, "out must be 16-byte aligned");
  const int64_t n = M * (L->d.H / 4);
  if (t_rc) t_rc->combine_blocks = ceil_div(n, kThreads);
  const dim3 grid((unsigned)ceil_div(n, kThreads));
  if (L->nloc < L->d.E)
    combine_kernel<true><<<grid, kThreads, 0, st>>>(at<uint2>(ws, lay.y), static_cast<uint2*>(out), (int)M, L->d.H,
                                                    L->d.top_k, (int)lay.T, (int)lay.S, at<int>(ws, lay.ids), L->lo,
                                                    L->nloc);
  else
    combine_kernel<false><<<grid, kThreads, 0, st>>>(at<uint2>(ws, lay.y), static_cast<uint2*>(out), (int)M, L->d.H,
                                                     L->d.top_k, (int)lay.T, (int)lay.S, nullptr, 0, L->nloc);
  return check_launch(L, "combine_kernel");
}

int do_router(qmoe_layer* L, const void* x, const void* w_router, int64_t M, float* logits, hipStream_t st) {
  if (!x || !w_router || !logits) return fail(QMOE_ERR_ARG, "x, w_router or logits is NULL");
  if (!aligned16(x) || !aligned16(w_router)) return fail(QMOE_ERR_ARG, "x and w_router must be 16-byte aligned");
  if ((int64_t)L->d.E * L->d.H * 2 >= (1LL << 31)) return fail(QMOE_ERR_UNSUPPORTED, "router weights too large");
  RouterArgs a;
  a.x = static_cast<const uint4*>(x);
  a.wr = static_cast<const uint4*>(w_router);
  a.logits = logits;
  a.M = (int)M;
  a.E = L->d.E;
  a.H = L->d.H;
  if (M <= kRouterGemvMaxM) {
    const int64_t waves = (int64_t)L->d.E * ceil_div(M, kRouterGemvTokens);
    router_gemv_kernel<<<dim3((unsigned)ceil_div(waves, kThreads / 64)), kThreads, 0, st>>>(a);
    return check_launch(L, "router_gemv_kernel");
  }
  const int64_t blocks = ceil_div(M, kRouterTok) * ceil_div(L->d.E, kRouterExp);
  router_tile_kernel<<<dim3((unsigned)blocks), kRouterThreads, 0, st>>>(a);
  return check_launch(L, "router_tile_kernel");
}

}  // namespace

// ================================================================ C ABI

extern "C" {

int qmoe_version(void) { return QMOE_VERSION; }

const char* qmoe_last_error(void) { return g_err.c_str(); }

namespace {
// The layer's codes and scales in tile order: w13 [L, 2I, H/2], w2
// [L, H, I/2] and their scales s13 [L, 2I, H/32], s2 [L, H, I/32] of the L
// local experts (and the shared expert's), copied once into one allocation,
// which the MFMA tiles read (the dot-product GEMV reads the caller's arrays
// as given).  The device is synchronised before (the caller's writes of the
// weights, on any stream, are complete) and after (the copy is complete
// before any stream can use it).
int make_tiled_weights(qmoe_layer* L) {
  const int64_t H = L->d.H, I = L->d.I, nl = L->nloc;
  if (hipDeviceSynchronize() != hipSuccess) return fail(QMOE_ERR_DEVICE, "hipDeviceSynchronize failed");
  const int64_t b13 = 2 * I * (H / 2), b2 = H * (I / 2);        // code bytes of one expert
  const int64_t c13 = 2 * I * (H / 32) * 2, c2 = H * (I / 32) * 2;  // scale bytes of one expert
  const int64_t nexp = nl + (L->shared ? 1 : 0);
  const int64_t total = nexp * (b13 + b2 + c13 + c2);
  if (hipMalloc(&L->tiled, (size_t)total) != hipSuccess) {
    L->tiled = nullptr;
    (void)hipGetLastError();
    return fail(QMOE_ERR_DEVICE, "cannot allocate " + std::to_string(total) + " bytes for the tile-ordered weights");
  }
  uint8_t* base = static_cast<uint8_t*>(L->tiled);
  uint8_t* sbase = base + nexp * (b13 + b2);  // the scales after all codes (16-byte aligned: b13, b2 are)
  struct Part {
    const void* src;
    uint8_t* dst;
    int64_t rows, K;
    bool scales;
  };
  const Part parts[8] = {{L->d.w13, base, nl * 2 * I, H, false},
                         {L->d.w2, base + nl * b13, nl * H, I, false},
                         {L->d.s13, sbase, nl * 2 * I, H, true},
                         {L->d.s2, sbase + nl * c13, nl * H, I, true},
                         {L->d.shared_w13, base + nl * (b13 + b2), 2 * I, H, false},
                         {L->d.shared_w2, base + nl * (b13 + b2) + b13, H, I, false},
                         {L->d.shared_s13, sbase + nl * (c13 + c2), 2 * I, H, true},
                         {L->d.shared_s2, sbase + nl * (c13 + c2) + c13, H, I, true}};
  for (int i = 0; i < (L->shared ? 8 : 4); ++i) {
    const Part& p = parts[i];
    if (p.scales) {
      const long long chunks = p.rows * (p.K / 32) / 4;
      tile_scales_kernel<<<dim3((unsigned)ceil_div(chunks, kThreads)), kThreads, 0, nullptr>>>(
          static_cast<const uint2*>(p.src), reinterpret_cast<uint2*>(p.dst), chunks, (int)(p.K / 32));
    } else {
      const long long chunks = p.rows * (p.K / 2) / 16;
      tile_codes_kernel<<<dim3((unsigned)ceil_div(chunks, kThreads)), kThreads, 0, nullptr>>>(
          static_cast<const uint4*>(p.src), reinterpret_cast<uint4*>(p.dst), chunks, (int)(p.K / 2));
    }
    if (hipGetLastError() != hipSuccess) return fail(QMOE_ERR_LAUNCH, "tiling the weights: launch failed");
  }
  if (hipDeviceSynchronize() != hipSuccess) return fail(QMOE_ERR_DEVICE, "tiling the weights failed");
  L->w13 = parts[0].dst;
  L->w2 = parts[1].dst;
  L->s13 = reinterpret_cast<const uint16_t*>(parts[2].dst);
  L->s2 = reinterpret_cast<const uint16_t*>(parts[3].dst);
  L->sh_w13 = L->shared ? parts[4].dst : nullptr;
  L->sh_w2 = L->shared ? parts[5].dst : nullptr;
  L->sh_s13 = L->shared ? reinterpret_cast<const uint16_t*>(parts[6].dst) : nullptr;
  L->sh_s2 = L->shared ? reinterpret_cast<const uint16_t*>(parts[7].dst) : nullptr;
  return QMOE_OK;
}
}  // namespace

int qmoe_layer_create(const qmoe_layer_desc* d, qmoe_layer** out) {
  if (!out) return fail(QMOE_ERR_ARG, "out is NULL");
  *out = nullptr;
  if (!d) return fail(QMOE_ERR_ARG, "desc is NULL");
  if (d->E < 1 || d->E > QMOE_MAX_EXPERTS) return fail(QMOE_ERR_ARG, "E must be in [1, 1024]");
  // a multiple of 128 keeps every row's scale quads 8-byte aligned
  if (d->H < 128 || d->H % 128) return fail(QMOE_ERR_ARG, "H must be a positive multiple of 128");
  if (d->I < 128 || d->I % 128) return fail(QMOE_ERR_ARG, "I must be a positive multiple of 128");
  if (d->top_k < 1 || d->top_k > d->E || d->top_k > QMOE_MAX_TOPK)
    return fail(QMOE_ERR_ARG, "top_k must be in [1, min(E, 32)]");
  if (d->group_size != QMOE_GROUP) return fail(QMOE_ERR_ARG, "group_size must be 32");
  if (d->max_rows < 1) return fail(QMOE_ERR_ARG, "max_rows must be >= 1");
  // activation buffers are addressed with 32-bit offsets
  if ((int64_t)d->max_rows * d->H * 2 >= (1LL << 31) ||
      (int64_t)d->max_rows * (d->top_k + 1) * d->I * 2 >= (1LL << 31))
    return fail(QMOE_ERR_ARG, "max_rows too large for 32-bit activation offsets");
  if ((int64_t)2 * d->I * d->H / 2 >= (1LL << 31)) return fail(QMOE_ERR_ARG, "expert too large");
  if (!d->w13) return fail(QMOE_ERR_ARG, "w13 is NULL");
  if (!d->s13) return fail(QMOE_ERR_ARG, "s13 is NULL");
  if (!d->w2) return fail(QMOE_ERR_ARG, "w2 is NULL");
  if (!d->s2) return fail(QMOE_ERR_ARG, "s2 is NULL");
  const int nsh = (d->shared_w13 != nullptr) + (d->shared_s13 != nullptr) + (d->shared_w2 != nullptr) +
                  (d->shared_s2 != nullptr);
  if (nsh != 0 && nsh != 4) return fail(QMOE_ERR_ARG, "shared expert: set all four pointers or none");
  if (!aligned16(d->w13) || !aligned16(d->w2) || (nsh && (!aligned16(d->shared_w13) || !aligned16(d->shared_w2))))
    return fail(QMOE_ERR_ARG, "weight code arrays must be 16-byte aligned");
  if (d->local_count < 0 || d->local_count > d->E || d->local_first < 0 ||
      (d->local_count > 0 && d->local_first > d->E - d->local_count))
    return fail(QMOE_ERR_ARG, "local experts [local_first, local_first + local_count) must lie in [0, E)");
  if (d->scoring != QMOE_SCORING_SOFTMAX && d->scoring != QMOE_SCORING_SIGMOID)
    return fail(QMOE_ERR_ARG, "scoring must be QMOE_SCORING_SOFTMAX or QMOE_SCORING_SIGMOID");
  if (d->expert_bias && d->scoring != QMOE_SCORING_SIGMOID)
    return fail(QMOE_ERR_ARG, "expert_bias is only for the sigmoid scoring");
  if (!(std::isfinite(d->routed_scale) && d->routed_scale >= 0.0f))
    return fail(QMOE_ERR_ARG, "routed_scale must be finite and >= 0 (0 means 1)");
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess) return fail(QMOE_ERR_DEVICE, "no HIP device (hipGetDevice failed)");
  hipDeviceProp_t prop;
  if (hipGetDeviceProperties(&prop, dev) != hipSuccess) return fail(QMOE_ERR_DEVICE, "hipGetDeviceProperties failed");
  if (std::strncmp(prop.gcnArchName, "gfx950", 6) != 0)
    return fail(QMOE_ERR_UNSUPPORTED, std::string("device arch ") + prop.gcnArchName + " is not gfx950");
  void* sp = nullptr;
  const hipError_t se = scratch_address(dev, &sp);
  if (se != hipSuccess)
    return fail(QMOE_ERR_DEVICE, std::string("hipGetSymbolAddress of the static scratch failed: ") + hipGetErrorString(se));
  qmoe_layer* L = new qmoe_layer;
  L->d = *d;
  L->device = dev;
  L->shared = nsh == 4;
  L->scratch = sp;
  L->lo = d->local_count ? d->local_first : 0;
  L->nloc = d->local_count ? d->local_count : d->E;
  L->rscale = d->routed_scale == 0.0f ? 1.0f : d->routed_scale;
  const int rc = make_tiled_weights(L);
  if (rc != QMOE_OK) {
    qmoe_layer_destroy(L);
    return rc;
  }
  *out = L;
  return QMOE_OK;
}

void qmoe_layer_destroy(qmoe_layer* L) {
  if (L && L->tiled) (void)hipFree(L->tiled);
  delete L;
}

int qmoe_workspace_size(const qmoe_layer* L, int64_t M, size_t* bytes) {
  if (!L || !bytes) return fail(QMOE_ERR_ARG, "layer or bytes is NULL");
  if (M < 0 || M > L->d.max_rows) return fail(QMOE_ERR_ARG, "M outside [0, max_rows]");
  *bytes = make_layout(L, M).total;
  return QMOE_OK;
}

int qmoe_workspace_init(qmoe_layer* L, void* ws, size_t ws_bytes, void* stream) {
  if (!L) return fail(QMOE_ERR_ARG, "layer is NULL");
  if (!ws) return fail(QMOE_ERR_WORKSPACE, "workspace is NULL");
  if (ws_bytes < kCtrlWords * 4) return fail(QMOE_ERR_WORKSPACE, "workspace too small");
  if ((reinterpret_cast<uintptr_t>(ws) & 255) != 0) return fail(QMOE_ERR_WORKSPACE, "workspace not 256-byte aligned");
  return init_workspace(L, ws, ws_bytes, static_cast<hipStream_t>(stream));
}

int qmoe_route(qmoe_layer* L, const void* x, const float* logits, int64_t M, void* ws, size_t ws_bytes,
               void* stream) {
  Layout lay;
  int rc = check_call(L, M, ws, ws_bytes, &lay);
  if (rc != QMOE_OK || M == 0) return rc;
  const hipStream_t st = static_cast<hipStream_t>(stream);
  return do_route(L, x, logits, M, ws, lay, st);
}

int qmoe_gate_up(qmoe_layer* L, int64_t M, void* ws, size_t ws_bytes, void* stream) {
  Layout lay;
  int rc = check_call(L, M, ws, ws_bytes, &lay);
  if (rc != QMOE_OK || M == 0) return rc;
  return do_gate_up(L, M, ws, lay, static_cast<hipStream_t>(stream));
}

int qmoe_down(qmoe_layer* L, int64_t M, void* ws, size_t ws_bytes, void* stream) {
  Layout lay;
  int rc = check_call(L, M, ws, ws_bytes, &lay);
  if (rc != QMOE_OK || M == 0) return rc;
  return do_down(L, M, ws, lay, static_cast<hipStream_t>(stream));
}

int qmoe_combine(qmoe_layer* L, int64_t M, void* out, void* ws, size_t ws_bytes, void* stream) {
  Layout lay;
  int rc = check_call(L, M, ws, ws_bytes, &lay);
  if (rc != QMOE_OK || M == 0) return rc;
  return do_combine(L, M, out, ws, lay, static_cast<hipStream_t>(stream));
}

namespace {
int forward_impl(qmoe_layer* L, const void* x, const float* logits, int64_t M, void* out, void* ws,
                 size_t ws_bytes, hipStream_t st, bool from_scratch) {
  Layout lay;
  int rc = check_call(L, M, ws, ws_bytes, &lay);
  if (rc != QMOE_OK || M == 0) return rc;
  if (!out) return fail(QMOE_ERR_ARG, "out is NULL");
  qmoe_receipt r{};
  r.M = M;
  const Regime rg = regime_of(L, M);
  r.regime = rg == kGemv ? QMOE_REGIME_GEMV : mixed_call(L, M) ? QMOE_REGIME_MIXED : QMOE_REGIME_TILES;
  r.rows_per_item = rows_per_item(rg);
  r.shared_expert = L->shared ? 1 : 0;
  r.route_kernels = lay.C == 1 ? 1 : 2;
  r.workspace_bytes = lay.total;
  r.static_scratch = from_scratch ? 1 : 0;
  r.splits_gate_up = r.splits_down = 1;
  t_rc = &r;
  if ((rc = do_route(L, x, logits, M, ws, lay, st)) == QMOE_OK && (rc = do_gate_up(L, M, ws, lay, st)) == QMOE_OK &&
      (rc = do_down(L, M, ws, lay, st)) == QMOE_OK)
    rc = do_combine(L, M, out, ws, lay, st);
  t_rc = nullptr;
  if (rc != QMOE_OK) return rc;
  L->forward_calls++;
  r.seq = ++L->receipt_seq;
  std::lock_guard<std::mutex> lock(L->receipt_mu);
  L->last = r;
  L->has_receipt = true;
  return QMOE_OK;
}
}  // namespace

int qmoe_forward(qmoe_layer* L, const void* x, const float* logits, int64_t M, void* out, void* ws,
                 size_t ws_bytes, void* stream) {
  return forward_impl(L, x, logits, M, out, ws, ws_bytes, static_cast<hipStream_t>(stream), false);
}

int qmoe_router_logits(qmoe_layer* L, const void* x, const void* w_router, int64_t M, float* logits,
                       void* stream) {
  if (!L) return fail(QMOE_ERR_ARG, "layer is NULL");
  if (M < 0 || M > L->d.max_rows) return fail(QMOE_ERR_ARG, "M outside [0, max_rows]");
  if (M == 0) return QMOE_OK;
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess || dev != L->device) return fail(QMOE_ERR_DEVICE, "not the layer's device");
  return do_router(L, x, w_router, M, logits, static_cast<hipStream_t>(stream));
}

int qmoe_forward_router(qmoe_layer* L, const void* x, const void* w_router, int64_t M, void* out, void* ws,
                        size_t ws_bytes, void* stream) {
  Layout lay;
  int rc = check_call(L, M, ws, ws_bytes, &lay);
  if (rc != QMOE_OK || M == 0) return rc;
  const hipStream_t st = static_cast<hipStream_t>(stream);
  float* logits = at<float>(ws, lay.logits);
  qmoe_receipt r0{};
  t_rc = &r0;  // the router launch counts toward the call's receipt
  rc = do_router(L, x, w_router, M, logits, st);
  t_rc = nullptr;
  if (rc != QMOE_OK) return rc;
  rc = forward_impl(L, x, logits, M, out, ws, ws_bytes, st, false);
  if (rc != QMOE_OK) return rc;
  std::lock_guard<std::mutex> lock(L->receipt_mu);
  L->last.launches += r0.launches;
  L->last.router = 1;
  return QMOE_OK;
}

int qmoe_last_receipt(const qmoe_layer* L, qmoe_receipt* out) {
  if (!L || !out) return fail(QMOE_ERR_ARG, "layer or receipt is NULL");
  std::lock_guard<std::mutex> lock(const_cast<qmoe_layer*>(L)->receipt_mu);
  if (!L->has_receipt) return fail(QMOE_ERR_ARG, "no forward call has completed on this layer");
  *out = L->last;
  return QMOE_OK;
}

int qmoe_read_item_count(qmoe_layer* L, int64_t M, const void* ws, size_t ws_bytes, int32_t* n_items, void* stream) {
  Layout lay;
  int rc = check_call(L, M, ws, ws_bytes, &lay);
  if (rc != QMOE_OK) return rc;
  if (!n_items) return fail(QMOE_ERR_ARG, "n_items is NULL");
  if (M == 0) return fail(QMOE_ERR_ARG, "M=0 builds no work list");
  if (hipMemcpyAsync(n_items, static_cast<const char*>(ws) + lay.ctrl + 4, 4, hipMemcpyDeviceToDevice,
                     static_cast<hipStream_t>(stream)) != hipSuccess)
    return fail(QMOE_ERR_LAUNCH, "hipMemcpyAsync of the item count failed");
  return QMOE_OK;
}

int qmoe_forward_static(qmoe_layer* L, const void* x, const float* logits, int64_t M, void* out, void* stream) {
  if (!L) return fail(QMOE_ERR_ARG, "layer is NULL");
  if (M < 0 || M > L->d.max_rows) return fail(QMOE_ERR_ARG, "M outside [0, max_rows]");
  const size_t need = make_layout(L, M).total;
  if (need > kScratchBytes)
    return fail(QMOE_ERR_WORKSPACE, "M=" + std::to_string(M) + " needs " + std::to_string(need) +
                                        " bytes of scratch, more than the static " + std::to_string(kScratchBytes));
  return forward_impl(L, x, logits, M, out, L->scratch, kScratchBytes, static_cast<hipStream_t>(stream), true);
}

int qmoe_read_routing(qmoe_layer* L, int64_t M, const void* ws, size_t ws_bytes, int32_t* ids, float* w,
                      int32_t* counts, int32_t* offsets, int32_t* perm, void* stream) {
  Layout lay;
  int rc = check_call(L, M, ws, ws_bytes, &lay);
  if (rc != QMOE_OK || M == 0) return rc;
  const hipStream_t st = static_cast<hipStream_t>(stream);
  const char* base = static_cast<const char*>(ws);
  struct Cp {
    void* dst;
    size_t off, bytes;
  } cps[] = {{ids, lay.ids, (size_t)lay.T * 4},
             {w, lay.wts, (size_t)lay.T * 4},
             {counts, lay.counts, (size_t)L->nloc * 4},
             {offsets, lay.offsets, (size_t)(L->nloc + 1) * 4},
             {perm, lay.perm, (size_t)lay.T * 4}};
  for (const Cp& c : cps) {
    if (!c.dst) continue;
    if (hipMemcpyAsync(c.dst, base + c.off, c.bytes, hipMemcpyDeviceToDevice, st) != hipSuccess)
      return fail(QMOE_ERR_LAUNCH, "hipMemcpyAsync of routing results failed");
  }
  return QMOE_OK;
}

int qmoe_read_intermediate(qmoe_layer* L, int64_t M, const void* ws, size_t ws_bytes, int32_t which,
                           float* out_f32, void* stream) {
  Layout lay;
  int rc = check_call(L, M, ws, ws_bytes, &lay);
  if (rc != QMOE_OK || M == 0) return rc;
  if (!out_f32) return fail(QMOE_ERR_ARG, "out_f32 is NULL");
  const hipStream_t st = static_cast<hipStream_t>(stream);
  void* w = const_cast<void*>(ws);
  if (which == 0) {
    const int64_t n = lay.R * L->d.I;
    read_h_kernel<<<dim3((unsigned)ceil_div(n, kThreads)), kThreads, 0, st>>>(
        at<_Float16>(w, lay.h), at<int>(w, lay.inv_perm), at<int>(w, lay.xexp), (int)lay.T, L->d.top_k, lay.R,
        L->d.I, out_f32);
    return check_launch(L, "read_h_kernel");
  }
  if (which == 1) {
    const int64_t n = lay.R * L->d.H;
    read_y_kernel<<<dim3((unsigned)ceil_div(n, kThreads)), kThreads, 0, st>>>(at<uint16_t>(w, lay.y), n, out_f32);
    return check_launch(L, "read_y_kernel");
  }
  return fail(QMOE_ERR_ARG, "which must be 0 (h) or 1 (y)");
}

int qmoe_dequant_debug(qmoe_layer* L, int32_t expert, int32_t which, uint16_t* out, void* stream) {
  if (!L) return fail(QMOE_ERR_ARG, "layer is NULL");
  if (!out) return fail(QMOE_ERR_ARG, "out is NULL");
  if (expert < 0 || expert > L->nloc || (expert == L->nloc && !L->shared))
    return fail(QMOE_ERR_ARG, "expert out of range");
  if (which != 0 && which != 1) return fail(QMOE_ERR_ARG, "which must be 0 (w13) or 1 (w2)");
  const int64_t H = L->d.H, I = L->d.I;
  const int N = which == 0 ? (int)(2 * I) : (int)H;
  const int K = which == 0 ? (int)H : (int)I;
  const uint8_t* w;
  const uint16_t* s;
  if (expert < L->nloc) {
    w = (which == 0 ? L->w13 : L->w2) + (size_t)expert * N * (K / 2);
    s = (which == 0 ? L->s13 : L->s2) + (size_t)expert * N * (K / 32);
  } else {
    w = which == 0 ? L->sh_w13 : L->sh_w2;
    s = which == 0 ? L->sh_s13 : L->sh_s2;
  }
  const int64_t n = (int64_t)N * (K / 8);
  dequant_kernel<<<dim3((unsigned)ceil_div(n, kThreads)), kThreads, 0, static_cast<hipStream_t>(stream)>>>(
      reinterpret_cast<const uint32_t*>(w), s, N, K, out);
  return check_launch(L, "dequant_kernel");
}

int qmoe_get_stats(const qmoe_layer* L, qmoe_stats* s) {
  if (!L || !s) return fail(QMOE_ERR_ARG, "layer or stats is NULL");
  s->forward_calls = L->forward_calls.load();
  s->route_calls = L->route_calls.load();
  s->gemm_launches = L->gemm_launches.load();
  s->launches = L->launches.load();
  s->workspace_inits = L->inits.load();
  s->workspace_bytes_last = L->ws_last.load();
  s->workspace_bytes_peak = L->ws_peak.load();
  s->prefill_tiles = L->prefill_tiles.load();
  s->gemv_tiles = L->gemv_tiles.load();
  s->gemv_nt_launches = L->gemv_nt.load();
  s->splitk_launches = L->splitk_launches.load();
  return QMOE_OK;
}

int qmoe_reset_stats(qmoe_layer* L) {
  if (!L) return fail(QMOE_ERR_ARG, "layer is NULL");
  L->forward_calls = 0;
  L->route_calls = 0;
  L->gemm_launches = 0;
  L->launches = 0;
  L->inits = 0;
  L->ws_last = 0;
  L->ws_peak = 0;
  L->prefill_tiles = 0;
  L->gemv_tiles = 0;
  L->gemv_nt = 0;
  L->splitk_launches = 0;
  return QMOE_OK;
}

}  // extern "C"
