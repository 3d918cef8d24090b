// Fused int4 group-32 Mixture-of-Experts layer for AMD Instinct MI355X
// (gfx950): HIP kernels and the host side of the C ABI declared in qmoe.h.
//
// Steps of one call, one kernel each, all on the caller's stream:
//   route_kernel    top-k routing, expert counts, their exclusive scan, the
//                   stable sort of routed slots by expert, the flat list of
//                   (expert, row tile) work items, x -> fp16 operand format
//   gemm_kernel<..., true>   stacked gate+up product with h = SiLU(g)*u
//   gemm_kernel<..., false>  down product times the routing weight
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
#include <cstring>
#include <mutex>
#include <string>
#include <utility>
#include <vector>

#include "qmoe.h"
#include "qmoe_device.h"

using namespace qmoe;

namespace {

constexpr int kThreads = 256;   // every kernel: 4 waves of 64
constexpr int kChunk = 64;      // tokens per routing chunk = bits of one mask word
constexpr int kCtrlWords = 64;  // [0] route ticket, [1] number of work items
constexpr int kKStep = 128;     // inputs per K-step of a wave (4 lane groups x 32)
constexpr int kAStride = kKStep + 8;  // LDS row stride of the A tile (halves), padded

// ---------------------------------------------------------------- routing

struct RouteArgs {
  const float* logits;
  const uint4* x;  // bf16 [M, H] as 16-byte runs
  int M, E, H, k, S, C, bmc, max_items;
  int* ctrl;
  int* ids;
  float* wts;
  int* counts;
  int* offsets;
  unsigned long long* cmask;  // [C, E] token bitmask per chunk and expert
  int* pbase;                 // [C, E] first sorted position of a chunk's tokens
  int* perm;
  int* inv_perm;
  int4* items;
  uint4* xa;  // fp16 A-format [M, H]
};

// Exclusive scan of in[0..n) into out[0..n] (out[n] = total) by the 256
// threads of a block: each thread sums 5 consecutive entries, a wave-wide
// Hillis-Steele scan over lanes combines them, then the 4 wave totals.
__device__ void block_exclusive_scan(const int* in, int* out, int n, int* wsum) {
  constexpr int kPer = 5;  // 256 * 5 >= QMOE_MAX_EXPERTS + 1
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  int v[kPer];
  int local = 0;
#pragma unroll
  for (int i = 0; i < kPer; ++i) {
    const int idx = tid * kPer + i;
    v[i] = idx < n ? in[idx] : 0;
    local += v[i];
  }
  int incl = local;
#pragma unroll
  for (int off = 1; off < 64; off <<= 1) {
    const int o = __shfl_up(incl, off, 64);
    if (lane >= off) incl += o;
  }
  if (lane == 63) wsum[wave] = incl;
  __syncthreads();
  int run = incl - local;
  for (int w = 0; w < wave; ++w) run += wsum[w];
#pragma unroll
  for (int i = 0; i < kPer; ++i) {
    const int idx = tid * kPer + i;
    if (idx < n) out[idx] = run;
    run += v[i];
  }
  if (tid == kThreads - 1) out[n] = run;
  __syncthreads();
}

// One block per chunk of 64 tokens; the last block to finish (atomic ticket,
// no waiting) turns the per-chunk masks into counts, offsets, positions and
// work items.  EPL = logits per lane (E <= 64 * EPL).
template <int EPL>
__global__ __launch_bounds__(kThreads) void route_kernel(RouteArgs a) {
  __shared__ uint32_t cm[QMOE_MAX_EXPERTS][2];
  __shared__ int s_cnt[QMOE_MAX_EXPERTS + 2];
  __shared__ int s_off[QMOE_MAX_EXPERTS + 2];
  __shared__ int s_ni[QMOE_MAX_EXPERTS + 2];
  __shared__ int s_ioff[QMOE_MAX_EXPERTS + 2];
  __shared__ int s_wsum[4];
  __shared__ int s_last;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int c = blockIdx.x, E = a.E, k = a.k;

  for (int e = tid; e < E; e += kThreads) cm[e][0] = cm[e][1] = 0u;
  __syncthreads();

  // ---- phase 1: each wave routes 16 tokens of the chunk
  for (int i = 0; i < kChunk / 4; ++i) {
    const int tl = wave * (kChunk / 4) + i;
    const int t = c * kChunk + tl;
    if (t >= a.M) break;
    const float* row = a.logits + (size_t)t * E;
    // key = (order-preserving logit bits, ~expert): the maximum key is the
    // largest logit, ties to the lowest expert index.  Absent experts = 0.
    uint64_t key[EPL];
#pragma unroll
    for (int s = 0; s < EPL; ++s) {
      const int e = s * 64 + lane;
      key[s] = (e < E) ? (((uint64_t)ordered_key(row[e]) << 32) | (uint32_t)(~e)) : 0ull;
    }
    int my_e = 0;
    for (int j = 0; j < k; ++j) {
      uint64_t best = 0;
#pragma unroll
      for (int s = 0; s < EPL; ++s) best = key[s] > best ? key[s] : best;
#pragma unroll
      for (int m = 32; m >= 1; m >>= 1) {
        const uint64_t o = shfl_xor_u64(best, m);
        best = o > best ? o : best;
      }
      const int e_sel = (int)(~(uint32_t)best);
#pragma unroll
      for (int s = 0; s < EPL; ++s)
        if (s * 64 + lane == e_sel) key[s] = 0;
      if (lane == j) my_e = e_sel;
    }
    // renormalised softmax over the selected logits: the full-softmax
    // denominator cancels, so w_j = exp(l_j - l_0) / sum_j' exp(l_j' - l_0)
    const float lj = (lane < k) ? row[my_e] : 0.0f;
    const float l0 = __shfl(lj, 0, 64);
    const float ex = (lane < k) ? expf(lj - l0) : 0.0f;
    float sum = ex;
#pragma unroll
    for (int m = 32; m >= 1; m >>= 1) sum += __shfl_xor(sum, m, 64);
    if (lane < k) {
      a.ids[(size_t)t * k + lane] = my_e;
      a.wts[(size_t)t * k + lane] = ex / sum;
      atomicOr(&cm[my_e][tl >> 5], 1u << (tl & 31));
    }
    // x row -> fp16 operand format
    const uint4* xs = a.x + (size_t)t * (a.H / 8);
    uint4* xd = a.xa + (size_t)t * (a.H / 8);
    for (int ch = lane; ch < a.H / 8; ch += 64) xd[ch] = bf16x8_to_aformat(xs[ch]);
  }
  __syncthreads();
  for (int e = tid; e < E; e += kThreads)
    a.cmask[(size_t)c * E + e] = (unsigned long long)cm[e][0] | ((unsigned long long)cm[e][1] << 32);
  __threadfence();
  __syncthreads();
  if (tid == 0) s_last = (atomicAdd(a.ctrl, 1) == a.C - 1);
  __syncthreads();
  if (!s_last) return;
  __threadfence();

  // ---- phase 2 (last block only)
  const int T = a.M * k;
  for (int e = tid; e < E; e += kThreads) {
    int n = 0;
    for (int cc = 0; cc < a.C; ++cc) n += __popcll(a.cmask[(size_t)cc * E + e]);
    s_cnt[e] = n;
  }
  if (tid == 0) s_cnt[E] = a.S;  // the shared expert takes every token
  __syncthreads();
  for (int e = tid; e <= E; e += kThreads) s_ni[e] = (s_cnt[e] + a.bmc - 1) / a.bmc;
  __syncthreads();
  block_exclusive_scan(s_cnt, s_off, E + 1, s_wsum);
  block_exclusive_scan(s_ni, s_ioff, E + 1, s_wsum);
  for (int e = tid; e <= E; e += kThreads) a.counts[e] = s_cnt[e];
  for (int e = tid; e <= E + 1; e += kThreads) a.offsets[e] = s_off[e];
  for (int e = tid; e < E; e += kThreads) {
    int run = s_off[e];
    for (int cc = 0; cc < a.C; ++cc) {
      a.pbase[(size_t)cc * E + e] = run;
      run += __popcll(a.cmask[(size_t)cc * E + e]);
    }
  }
  for (int e = tid; e <= E; e += kThreads) {
    const int base = s_ioff[e], n = s_cnt[e];
    for (int i = 0; i < s_ni[e]; ++i) {
      const int r0 = i * a.bmc;
      if (base + i < a.max_items) a.items[base + i] = make_int4(e, r0, min(a.bmc, n - r0), s_off[e] + r0);
    }
  }
  if (tid == 0) a.ctrl[1] = min(s_ioff[E + 1], a.max_items);
  __threadfence();
  __syncthreads();
  for (int f = tid; f < T; f += kThreads) {
    const int t = f / k, e = a.ids[f];
    const int cc = t / kChunk, tl = t % kChunk;
    const unsigned long long m = a.cmask[(size_t)cc * E + e];
    const int rank = __popcll(m & ((1ull << tl) - 1ull));
    const int pos = a.pbase[(size_t)cc * E + e] + rank;
    a.perm[pos] = f;
    a.inv_perm[f] = pos;
  }
  for (int t = tid; t < a.S; t += kThreads) a.perm[T + t] = T + t;
  __syncthreads();
  if (tid == 0) atomicExch(a.ctrl, 0);
}

// ------------------------------------------------------------------ GEMMs

struct GemmArgs {
  const uint8_t* w;    // routed experts' codes  [E, Nw, K/2]
  const uint16_t* s;   // routed experts' scales [E, Nw, K/32]
  const uint8_t* w_sh; // shared expert (may be null)
  const uint16_t* s_sh;
  int E, K, N, Nw, nblk, max_items, T, k, M, R;
  const int* ctrl;
  const int4* items;
  const int* perm;
  const float* wts;
  const _Float16* a;  // A rows in A-format: x (gate+up) or h (down)
  _Float16* h_out;    // gate+up: h [R, N] in A-format
  float* y_out;       // down: y [R, N] in slot order
};

template <int NBB, int MB>
struct Frag {
  uint4 b[NBB];       // 32 packed codes of this lane's weight row per block
  uint32_t sc[NBB];   // the group's fp16 scale bits
};

__device__ __forceinline__ uint32_t word(const uint4& v, int i) {
  return i == 0 ? v.x : i == 1 ? v.y : i == 2 ? v.z : v.w;
}

// One work item = (expert, up to MB*16 routed rows) x (an N range).  A block
// has 4 waves: WN waves along N (each NBW blocks of 16 output columns) times
// WK waves along K (partial sums reduced through LDS in a fixed order).
// Per K-step a lane of group kq (= lane/16) decodes the 32 codes of inputs
// [k0 + 32kq, +32) of one weight row: one 16-byte load and one scale.
// MB == 1: A rows are read straight from global memory (decode, few rows);
// MB > 1: the block stages the A tile for each K-step in LDS.
template <int MB, int NBW, int WN, int WK, bool GATEUP>
__global__ __launch_bounds__(kThreads) void gemm_kernel(GemmArgs g) {
  static_assert(WN * WK == 4, "4 waves per block");
  constexpr int NBB = GATEUP ? 2 * NBW : NBW;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int wn = wave % WN, wk = wave / WN;
  const int r = lane & 15, kq = lane >> 4;

  // all blocks of one item land on one XCD (block ids go round-robin over 8)
  const int bid = blockIdx.x, xcd = bid & 7, jj = bid >> 3;
  const int item = (jj / g.nblk) * 8 + xcd, nb = jj % g.nblk;
  const int n_items = min(g.ctrl[1], g.max_items);
  if (item >= n_items) return;
  const int4 it = g.items[item];
  const int e = it.x, nr = it.z, pos0 = it.w;
  // work items come from the workspace: reject any that do not fit it
  if (e < 0 || e > g.E || nr <= 0 || nr > MB * 16 || pos0 < 0 || pos0 > g.R - nr) return;
  const size_t K2 = (size_t)g.K / 2, KG = (size_t)g.K / 32;
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

  // weight rows of this lane, per B block
  const uint8_t* brow[NBB];
  const uint16_t* srow[NBB];
  int col0[NBW];
#pragma unroll
  for (int c = 0; c < NBW; ++c) {
    col0[c] = ((nb * WN + wn) * NBW + c) * 16;
    const int n = col0[c] < g.N ? col0[c] + r : 0;
    if (GATEUP) {
      brow[2 * c] = wb + (size_t)n * K2;
      srow[2 * c] = sbase + (size_t)n * KG;
      brow[2 * c + 1] = wb + (size_t)(g.N + n) * K2;
      srow[2 * c + 1] = sbase + (size_t)(g.N + n) * KG;
    } else {
      brow[c] = wb + (size_t)n * K2;
      srow[c] = sbase + (size_t)n * KG;
    }
  }

  const int nsteps = (g.K + kKStep - 1) / kKStep;
  const int s_begin = wk * nsteps / WK, s_end = (wk + 1) * nsteps / WK;
  const int nmb = (nr + 15) / 16;

  float4_t acc[MB][NBB];
#pragma unroll
  for (int mb = 0; mb < MB; ++mb)
#pragma unroll
    for (int b = 0; b < NBB; ++b) acc[mb][b] = float4_t{0.f, 0.f, 0.f, 0.f};

  auto load_b = [&](int s, Frag<NBB, MB>& f) {
    const int kk = s * kKStep + 32 * kq;
    const bool kv = kk < g.K;
#pragma unroll
    for (int b = 0; b < NBB; ++b) {
      f.b[b] = kv ? *reinterpret_cast<const uint4*>(brow[b] + kk / 2)
                  : make_uint4(0x88888888u, 0x88888888u, 0x88888888u, 0x88888888u);
      f.sc[b] = kv ? (uint32_t)srow[b][kk / 32] : 0u;
    }
  };

  // A source row (element offset of the row start) of tile row m, -1 if absent
  auto a_row_of = [&](int m) -> long long {
    if (m >= nr) return -1;
    const int pos = pos0 + m;
    if (GATEUP) {
      const int slot = g.perm[pos];
      if (slot < 0 || slot >= g.R) return -1;
      const int tok = slot < g.T ? slot / g.k : slot - g.T;
      if (tok >= g.M) return -1;
      return (long long)tok * g.K;
    }
    return (long long)pos * g.K;
  };

  if constexpr (MB == 1) {
    // ---------------- decode tiles: A straight from global memory
    const long long arow = a_row_of(r);
    uint4 aq[4], aqn[4];
    Frag<NBB, MB> f, fn;
    auto load_a = [&](int s, uint4 (&q)[4]) {
      const int kk = s * kKStep + 32 * kq;
      const bool ok = arow >= 0 && kk < g.K;
      const uint4* p = reinterpret_cast<const uint4*>(g.a + (ok ? arow + kk : 0));
#pragma unroll
      for (int i = 0; i < 4; ++i) q[i] = ok ? p[i] : make_uint4(0u, 0u, 0u, 0u);
    };
    if (s_begin < s_end) {
      load_b(s_begin, f);
      load_a(s_begin, aq);
    }
    for (int s = s_begin; s < s_end; ++s) {
      if (s + 1 < s_end) {
        load_b(s + 1, fn);
        load_a(s + 1, aqn);
      }
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const half8_t av = __builtin_bit_cast(half8_t, aq[i]);
#pragma unroll
        for (int b = 0; b < NBB; ++b) acc[0][b] = mfma16x16x32(av, dq8(word(f.b[b], i), f.sc[b]), acc[0][b]);
      }
      f = fn;
#pragma unroll
      for (int i = 0; i < 4; ++i) aq[i] = aqn[i];
    }
  } else {
    // ---------------- prefill tiles: A tile of the K-step staged in LDS
    __shared__ __attribute__((aligned(16))) _Float16 lds_a[MB * 16 * kAStride];
    __shared__ long long lds_row[MB * 16];
    for (int m = tid; m < MB * 16; m += kThreads) lds_row[m] = a_row_of(m);
    __syncthreads();
    // thread -> 16-byte segment `seg` of rows (tid/16) + 16*i of the tile
    const int seg = tid & 15, row_base = tid >> 4;
    constexpr int kRowsPerThread = MB;  // MB*16 rows / 16 row groups
    uint4 st[kRowsPerThread];
    auto load_a_tile = [&](int s) {
      const int kk = s * kKStep + seg * 8;
#pragma unroll
      for (int i = 0; i < kRowsPerThread; ++i) {
        const long long ar = lds_row[row_base + 16 * i];
        st[i] = (ar >= 0 && kk < g.K) ? *reinterpret_cast<const uint4*>(g.a + ar + kk)
                                      : make_uint4(0u, 0u, 0u, 0u);
      }
    };
    Frag<NBB, MB> f, fn;
    // every wave of the block runs the same K range here (WK == 1 for MB > 1)
    if (s_begin < s_end) {
      load_b(s_begin, f);
      load_a_tile(s_begin);
    }
    for (int s = s_begin; s < s_end; ++s) {
      __syncthreads();
#pragma unroll
      for (int i = 0; i < kRowsPerThread; ++i)
        *reinterpret_cast<uint4*>(&lds_a[(row_base + 16 * i) * kAStride + seg * 8]) = st[i];
      __syncthreads();
      if (s + 1 < s_end) {
        load_b(s + 1, fn);
        load_a_tile(s + 1);
      }
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        half8_t bf[NBB];
#pragma unroll
        for (int b = 0; b < NBB; ++b) bf[b] = dq8(word(f.b[b], i), f.sc[b]);
#pragma unroll
        for (int mb = 0; mb < MB; ++mb) {
          if (mb < nmb) {
            const half8_t av =
                *reinterpret_cast<const half8_t*>(&lds_a[(mb * 16 + r) * kAStride + 32 * kq + 8 * i]);
#pragma unroll
            for (int b = 0; b < NBB; ++b) acc[mb][b] = mfma16x16x32(av, bf[b], acc[mb][b]);
          }
        }
      }
      f = fn;
    }
  }

  // ---- reduce the WK partial sums (fixed order: wave wk=0 adds 1, 2, 3)
  if constexpr (WK > 1) {
    constexpr int kVals = MB * NBB * 4;
    __shared__ float red[(WK - 1) * WN * kVals * 64];
    if (wk > 0) {
#pragma unroll
      for (int mb = 0; mb < MB; ++mb)
#pragma unroll
        for (int b = 0; b < NBB; ++b)
#pragma unroll
          for (int i = 0; i < 4; ++i)
            red[((((wk - 1) * WN + wn) * kVals) + (mb * NBB + b) * 4 + i) * 64 + lane] = acc[mb][b][i];
    }
    __syncthreads();
    if (wk > 0) return;
#pragma unroll
    for (int w = 1; w < WK; ++w)
#pragma unroll
      for (int mb = 0; mb < MB; ++mb)
#pragma unroll
        for (int b = 0; b < NBB; ++b)
#pragma unroll
          for (int i = 0; i < 4; ++i)
            acc[mb][b][i] += red[((((w - 1) * WN + wn) * kVals) + (mb * NBB + b) * 4 + i) * 64 + lane];
  }

  // ---- epilogue: lane holds rows mb*16 + 4*kq + i of column r of each block
#pragma unroll
  for (int c = 0; c < NBW; ++c) {
    if (col0[c] >= g.N) continue;
    const int col = col0[c] + r;
#pragma unroll
    for (int mb = 0; mb < MB; ++mb) {
      if (mb >= nmb) continue;
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int row = mb * 16 + 4 * kq + i;
        if (row >= nr) continue;
        const int pos = pos0 + row;
        if (GATEUP) {
          const float gt = acc[mb][2 * c][i], up = acc[mb][2 * c + 1][i];
          const float hv = gt / (1.0f + __expf(-gt)) * up;
          g.h_out[(size_t)pos * g.N + ((col & ~7) | inv_perm8(col & 7))] = (_Float16)hv;
        } else {
          const int slot = g.perm[pos];
          if (slot < 0 || slot >= g.R) continue;
          const float wv = slot < g.T ? g.wts[slot] : 1.0f;
          g.y_out[(size_t)slot * g.N + col] = wv * acc[mb][c][i];
        }
      }
    }
  }
}

// ---------------------------------------------------------------- combine

// out[t, n] = sum_{j<k} y[t*k + j, n] (in j order) + y[T + t, n] if shared,
// rounded to bf16.  One thread per 8 consecutive columns.
__global__ __launch_bounds__(kThreads) void combine_kernel(const float* y, uint4* out, int M, int H,
                                                            int k, int T, int S) {
  const long long q = (long long)blockIdx.x * kThreads + threadIdx.x;
  const int per_row = H / 8;
  if (q >= (long long)M * per_row) return;
  const int t = (int)(q / per_row), c8 = (int)(q % per_row);
  float acc[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
  for (int j = 0; j < k; ++j) {
    const float4* p = reinterpret_cast<const float4*>(y + ((size_t)t * k + j) * H + (size_t)c8 * 8);
    const float4 u = p[0], v = p[1];
    acc[0] += u.x; acc[1] += u.y; acc[2] += u.z; acc[3] += u.w;
    acc[4] += v.x; acc[5] += v.y; acc[6] += v.z; acc[7] += v.w;
  }
  if (S) {
    const float4* p = reinterpret_cast<const float4*>(y + ((size_t)T + t) * H + (size_t)c8 * 8);
    const float4 u = p[0], v = p[1];
    acc[0] += u.x; acc[1] += u.y; acc[2] += u.z; acc[3] += u.w;
    acc[4] += v.x; acc[5] += v.y; acc[6] += v.z; acc[7] += v.w;
  }
  uint4 o;
  o.x = f32_to_bf16_rne(acc[0]) | (f32_to_bf16_rne(acc[1]) << 16);
  o.y = f32_to_bf16_rne(acc[2]) | (f32_to_bf16_rne(acc[3]) << 16);
  o.z = f32_to_bf16_rne(acc[4]) | (f32_to_bf16_rne(acc[5]) << 16);
  o.w = f32_to_bf16_rne(acc[6]) | (f32_to_bf16_rne(acc[7]) << 16);
  out[q] = o;
}

// ------------------------------------------------------------- inspection

__global__ __launch_bounds__(kThreads) void dequant_kernel(const uint32_t* w, const uint16_t* s, int N,
                                                            int K, uint16_t* out) {
  const long long idx = (long long)blockIdx.x * kThreads + threadIdx.x;
  const int per_row = K / 8;
  if (idx >= (long long)N * per_row) return;
  const int n = (int)(idx / per_row), d = (int)(idx % per_row);
  // bit-cast the whole vector (a bit-cast of one vector element reads element 0)
  const u16x8_t h = __builtin_bit_cast(u16x8_t, dq8(w[idx], s[(size_t)n * (K / 32) + d / 4]));
#pragma unroll
  for (int p = 0; p < 8; ++p) out[(size_t)n * K + d * 8 + perm8(p)] = h[p];
}

__global__ __launch_bounds__(kThreads) void read_h_kernel(const _Float16* h, const int* inv_perm, int T,
                                                           long long R, int I, float* out) {
  const long long q = (long long)blockIdx.x * kThreads + threadIdx.x;
  if (q >= R * I) return;
  const long long f = q / I;
  const int col = (int)(q % I);
  long long pos = f < T ? inv_perm[f] : f;
  if (pos < 0 || pos >= R) pos = f;
  out[q] = (float)h[pos * I + ((col & ~7) | inv_perm8(col & 7))];
}

__global__ void init_ctrl_kernel(int* ctrl) {
  if (threadIdx.x < kCtrlWords) ctrl[threadIdx.x] = 0;
}

// ============================================================= host side

thread_local std::string g_err;

int fail(int code, const std::string& msg) {
  g_err = msg;
  return code;
}

size_t align256(size_t v) { return (v + 255) & ~(size_t)255; }

struct Layout {
  int64_t T, S, R, C, max_items16;
  size_t ctrl, ids, wts, counts, offsets, cmask, pbase, perm, inv_perm, items, xa, h, y, total;
};

int64_t ceil_div(int64_t a, int64_t b) { return (a + b - 1) / b; }

int64_t max_items_for(int64_t T, int64_t M, int64_t S, int64_t E, int64_t bmc) {
  return T / bmc + std::min<int64_t>(E, T) + (S ? ceil_div(M, bmc) : 0);
}

}  // namespace

struct qmoe_layer {
  qmoe_layer_desc d;
  int device = 0;
  bool shared = false;
  std::atomic<uint64_t> forward_calls{0}, route_calls{0}, gemm_launches{0}, launches{0}, inits{0},
      ws_last{0}, ws_peak{0}, decode_tiles{0}, prefill_tiles{0};
  std::mutex mu;
  std::vector<std::pair<const void*, size_t>> inited;
};

namespace {

Layout make_layout(const qmoe_layer* L, int64_t M) {
  Layout l{};
  const int64_t E = L->d.E, H = L->d.H, I = L->d.I, k = L->d.top_k;
  l.T = M * k;
  l.S = L->shared ? M : 0;
  l.R = l.T + l.S;
  l.C = ceil_div(M, kChunk);
  l.max_items16 = max_items_for(l.T, M, l.S, E, 16);
  size_t off = 0;
  auto take = [&](size_t bytes) {
    const size_t o = off;
    off = align256(off + bytes);
    return o;
  };
  l.ctrl = take(kCtrlWords * 4);
  l.ids = take(l.T * 4);
  l.wts = take(l.T * 4);
  l.counts = take((E + 1) * 4);
  l.offsets = take((E + 2) * 4);
  l.cmask = take(l.C * E * 8);
  l.pbase = take(l.C * E * 4);
  l.perm = take(l.R * 4);
  l.inv_perm = take(l.T * 4);
  l.items = take(l.max_items16 * 16);
  l.xa = take(M * H * 2);
  l.h = take(l.R * I * 2);
  l.y = take(l.R * H * 4);
  l.total = off;
  return l;
}

bool use_decode_tiles(const qmoe_layer* L, int64_t M) {
  return M * (int64_t)L->d.top_k < 8 * (int64_t)L->d.E;
}

template <typename T>
T* at(void* ws, size_t off) {
  return reinterpret_cast<T*>(static_cast<char*>(ws) + off);
}

int check_launch(qmoe_layer* L, const char* what) {
  L->launches++;
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
  init_ctrl_kernel<<<1, 64, 0, st>>>(static_cast<int*>(ws));
  L->inits++;
  const int rc = check_launch(L, "workspace init");
  if (rc != QMOE_OK) return rc;
  std::lock_guard<std::mutex> g(L->mu);
  L->inited.emplace_back(ws, ws_bytes);
  return QMOE_OK;
}

int ensure_inited(qmoe_layer* L, void* ws, size_t ws_bytes, hipStream_t st) {
  {
    std::lock_guard<std::mutex> g(L->mu);
    for (auto& p : L->inited)
      if (p.first == ws) return QMOE_OK;
  }
  return init_workspace(L, ws, ws_bytes, st);
}

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15) == 0; }

int do_route(qmoe_layer* L, const void* x, const float* logits, int64_t M, void* ws, const Layout& lay,
             hipStream_t st) {
  if (!x || !logits) return fail(QMOE_ERR_ARG, x ? "logits is NULL" : "x is NULL");
  if (!aligned16(x)) return fail(QMOE_ERR_ARG, "x must be 16-byte aligned");
  const bool dec = use_decode_tiles(L, M);
  const int bmc = dec ? 16 : 128;
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
  a.max_items = (int)max_items_for(lay.T, M, lay.S, L->d.E, bmc);
  a.ctrl = at<int>(ws, lay.ctrl);
  a.ids = at<int>(ws, lay.ids);
  a.wts = at<float>(ws, lay.wts);
  a.counts = at<int>(ws, lay.counts);
  a.offsets = at<int>(ws, lay.offsets);
  a.cmask = at<unsigned long long>(ws, lay.cmask);
  a.pbase = at<int>(ws, lay.pbase);
  a.perm = at<int>(ws, lay.perm);
  a.inv_perm = at<int>(ws, lay.inv_perm);
  a.items = at<int4>(ws, lay.items);
  a.xa = at<uint4>(ws, lay.xa);
  const dim3 grid((unsigned)lay.C);
  const int epl = (L->d.E + 63) / 64;
  if (epl <= 1) route_kernel<1><<<grid, kThreads, 0, st>>>(a);
  else if (epl <= 2) route_kernel<2><<<grid, kThreads, 0, st>>>(a);
  else if (epl <= 4) route_kernel<4><<<grid, kThreads, 0, st>>>(a);
  else if (epl <= 8) route_kernel<8><<<grid, kThreads, 0, st>>>(a);
  else route_kernel<16><<<grid, kThreads, 0, st>>>(a);
  L->route_calls++;
  return check_launch(L, "route_kernel");
}

template <int MB, int NBW, int WN, int WK, bool GATEUP>
int launch_gemm(qmoe_layer* L, int64_t M, void* ws, const Layout& lay, hipStream_t st) {
  GemmArgs g;
  const int E = L->d.E, H = L->d.H, I = L->d.I;
  g.E = E;
  g.T = (int)lay.T;
  g.M = (int)M;
  g.R = (int)lay.R;
  g.k = L->d.top_k;
  g.ctrl = at<int>(ws, lay.ctrl);
  g.items = at<int4>(ws, lay.items);
  g.perm = at<int>(ws, lay.perm);
  g.wts = at<float>(ws, lay.wts);
  if (GATEUP) {
    g.w = L->d.w13;
    g.s = L->d.s13;
    g.w_sh = L->d.shared_w13;
    g.s_sh = L->d.shared_s13;
    g.K = H;
    g.N = I;
    g.Nw = 2 * I;
    g.a = at<_Float16>(ws, lay.xa);
    g.h_out = at<_Float16>(ws, lay.h);
    g.y_out = nullptr;
  } else {
    g.w = L->d.w2;
    g.s = L->d.s2;
    g.w_sh = L->d.shared_w2;
    g.s_sh = L->d.shared_s2;
    g.K = I;
    g.N = H;
    g.Nw = H;
    g.a = at<_Float16>(ws, lay.h);
    g.h_out = nullptr;
    g.y_out = at<float>(ws, lay.y);
  }
  const int bmc = MB * 16;
  g.max_items = (int)max_items_for(lay.T, M, lay.S, E, bmc);
  g.nblk = (int)ceil_div(g.N, WN * NBW * 16);
  const int64_t blocks = 8 * (int64_t)g.nblk * ceil_div(g.max_items, 8);
  if (blocks > 0x7FFFFFFF) return fail(QMOE_ERR_UNSUPPORTED, "grid too large");
  gemm_kernel<MB, NBW, WN, WK, GATEUP><<<dim3((unsigned)blocks), kThreads, 0, st>>>(g);
  L->gemm_launches++;
  return check_launch(L, GATEUP ? "gate_up gemm" : "down gemm");
}

int do_gate_up(qmoe_layer* L, int64_t M, void* ws, const Layout& lay, hipStream_t st) {
  if (use_decode_tiles(L, M)) {
    L->decode_tiles++;
    return launch_gemm<1, 1, 1, 4, true>(L, M, ws, lay, st);
  }
  L->prefill_tiles++;
  return launch_gemm<8, 2, 4, 1, true>(L, M, ws, lay, st);
}

int do_down(qmoe_layer* L, int64_t M, void* ws, const Layout& lay, hipStream_t st) {
  if (use_decode_tiles(L, M)) return launch_gemm<1, 1, 4, 1, false>(L, M, ws, lay, st);
  return launch_gemm<8, 4, 4, 1, false>(L, M, ws, lay, st);
}

int do_combine(qmoe_layer* L, int64_t M, void* out, void* ws, const Layout& lay, hipStream_t st) {
  if (!out) return fail(QMOE_ERR_ARG, "out is NULL");
  if (!aligned16(out)) return fail(QMOE_ERR_ARG, "out must be 16-byte aligned");
  const int64_t n = M * (L->d.H / 8);
  combine_kernel<<<dim3((unsigned)ceil_div(n, kThreads)), kThreads, 0, st>>>(
      at<float>(ws, lay.y), static_cast<uint4*>(out), (int)M, L->d.H, L->d.top_k, (int)lay.T, (int)lay.S);
  return check_launch(L, "combine_kernel");
}

}  // namespace

// ================================================================ C ABI

extern "C" {

int qmoe_version(void) { return QMOE_VERSION; }

const char* qmoe_last_error(void) { return g_err.c_str(); }

int qmoe_layer_create(const qmoe_layer_desc* d, qmoe_layer** out) {
  if (!out) return fail(QMOE_ERR_ARG, "out is NULL");
  *out = nullptr;
  if (!d) return fail(QMOE_ERR_ARG, "desc is NULL");
  if (d->E < 1 || d->E > QMOE_MAX_EXPERTS) return fail(QMOE_ERR_ARG, "E must be in [1, 1024]");
  if (d->H < 32 || d->H % 32) return fail(QMOE_ERR_ARG, "H must be a positive multiple of 32");
  if (d->I < 32 || d->I % 32) return fail(QMOE_ERR_ARG, "I must be a positive multiple of 32");
  if (d->top_k < 1 || d->top_k > d->E || d->top_k > QMOE_MAX_TOPK)
    return fail(QMOE_ERR_ARG, "top_k must be in [1, min(E, 32)]");
  if (d->group_size != QMOE_GROUP) return fail(QMOE_ERR_ARG, "group_size must be 32");
  if (d->max_rows < 1) return fail(QMOE_ERR_ARG, "max_rows must be >= 1");
  if ((int64_t)d->max_rows * d->top_k > (1LL << 30) || (int64_t)d->max_rows * d->H > (1LL << 40))
    return fail(QMOE_ERR_ARG, "max_rows too large");
  if (!d->w13) return fail(QMOE_ERR_ARG, "w13 is NULL");
  if (!d->s13) return fail(QMOE_ERR_ARG, "s13 is NULL");
  if (!d->w2) return fail(QMOE_ERR_ARG, "w2 is NULL");
  if (!d->s2) return fail(QMOE_ERR_ARG, "s2 is NULL");
  const int nsh = (d->shared_w13 != nullptr) + (d->shared_s13 != nullptr) + (d->shared_w2 != nullptr) +
                  (d->shared_s2 != nullptr);
  if (nsh != 0 && nsh != 4) return fail(QMOE_ERR_ARG, "shared expert: set all four pointers or none");
  if (!aligned16(d->w13) || !aligned16(d->w2) || (nsh && (!aligned16(d->shared_w13) || !aligned16(d->shared_w2))))
    return fail(QMOE_ERR_ARG, "weight code arrays must be 16-byte aligned");
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess) return fail(QMOE_ERR_DEVICE, "no HIP device (hipGetDevice failed)");
  hipDeviceProp_t prop;
  if (hipGetDeviceProperties(&prop, dev) != hipSuccess) return fail(QMOE_ERR_DEVICE, "hipGetDeviceProperties failed");
  if (std::strncmp(prop.gcnArchName, "gfx950", 6) != 0)
    return fail(QMOE_ERR_UNSUPPORTED, std::string("device arch ") + prop.gcnArchName + " is not gfx950");
  qmoe_layer* L = new qmoe_layer;
  L->d = *d;
  L->device = dev;
  L->shared = nsh == 4;
  *out = L;
  return QMOE_OK;
}

void qmoe_layer_destroy(qmoe_layer* L) { delete L; }

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
  if ((rc = ensure_inited(L, ws, ws_bytes, st)) != QMOE_OK) return rc;
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

int qmoe_forward(qmoe_layer* L, const void* x, const float* logits, int64_t M, void* out, void* ws,
                 size_t ws_bytes, void* stream) {
  Layout lay;
  int rc = check_call(L, M, ws, ws_bytes, &lay);
  if (rc != QMOE_OK || M == 0) return rc;
  if (!out) return fail(QMOE_ERR_ARG, "out is NULL");
  const hipStream_t st = static_cast<hipStream_t>(stream);
  if ((rc = ensure_inited(L, ws, ws_bytes, st)) != QMOE_OK) return rc;
  if ((rc = do_route(L, x, logits, M, ws, lay, st)) != QMOE_OK) return rc;
  if ((rc = do_gate_up(L, M, ws, lay, st)) != QMOE_OK) return rc;
  if ((rc = do_down(L, M, ws, lay, st)) != QMOE_OK) return rc;
  if ((rc = do_combine(L, M, out, ws, lay, st)) != QMOE_OK) return rc;
  L->forward_calls++;
  return QMOE_OK;
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
             {counts, lay.counts, (size_t)L->d.E * 4},
             {offsets, lay.offsets, (size_t)(L->d.E + 1) * 4},
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
        at<_Float16>(w, lay.h), at<int>(w, lay.inv_perm), (int)lay.T, lay.R, L->d.I, out_f32);
    return check_launch(L, "read_h_kernel");
  }
  if (which == 1) {
    if (hipMemcpyAsync(out_f32, at<float>(w, lay.y), (size_t)lay.R * L->d.H * 4, hipMemcpyDeviceToDevice, st) !=
        hipSuccess)
      return fail(QMOE_ERR_LAUNCH, "hipMemcpyAsync of y failed");
    return QMOE_OK;
  }
  return fail(QMOE_ERR_ARG, "which must be 0 (h) or 1 (y)");
}

int qmoe_dequant_debug(qmoe_layer* L, int32_t expert, int32_t which, uint16_t* out, void* stream) {
  if (!L) return fail(QMOE_ERR_ARG, "layer is NULL");
  if (!out) return fail(QMOE_ERR_ARG, "out is NULL");
  if (expert < 0 || expert > L->d.E || (expert == L->d.E && !L->shared))
    return fail(QMOE_ERR_ARG, "expert out of range");
  if (which != 0 && which != 1) return fail(QMOE_ERR_ARG, "which must be 0 (w13) or 1 (w2)");
  const int64_t H = L->d.H, I = L->d.I;
  const int N = which == 0 ? (int)(2 * I) : (int)H;
  const int K = which == 0 ? (int)H : (int)I;
  const uint8_t* w;
  const uint16_t* s;
  if (expert < L->d.E) {
    w = (which == 0 ? L->d.w13 : L->d.w2) + (size_t)expert * N * (K / 2);
    s = (which == 0 ? L->d.s13 : L->d.s2) + (size_t)expert * N * (K / 32);
  } else {
    w = which == 0 ? L->d.shared_w13 : L->d.shared_w2;
    s = which == 0 ? L->d.shared_s13 : L->d.shared_s2;
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
  s->decode_tiles = L->decode_tiles.load();
  s->prefill_tiles = L->prefill_tiles.load();
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
  L->decode_tiles = 0;
  L->prefill_tiles = 0;
  return QMOE_OK;
}

}  // extern "C"
