/*
 * qmoe.h -- C ABI of a fused Mixture-of-Experts layer over 4-bit
 * group-quantized expert weights, for AMD Instinct MI355X (gfx950).
 *
 * The layer (definition: "The MoE Throughput Lever: Quantifying the INT4
 * Marlin GEMM on Blackwell PRO 6000", sections "The Context: Why This
 * Measurement Matters" and "The Benchmark: What Was Measured"; routing
 * counts: "Detailed results", section "Nsight Compute on the stock kernel";
 * sorted routing and the stacked gate+up GEMM: "perf(exl3): accelerate
 * fat-expert prefill", description and section "Rollout"):
 *
 *   for each token t of M:
 *     ids[t, 0..k-1] = the top_k experts by router logit (descending,
 *                      ties to the lower expert index)
 *     w[t, j]        = softmax(logits[t])[ids[t,j]], renormalised over j
 *                      (the default scoring; qmoe_layer_desc.scoring below
 *                      selects the sigmoid router instead)
 *     out[t]         = sum_j w[t,j] * Down_e( SiLU(Gate_e x_t) * (Up_e x_t) ),
 *                      e = ids[t,j], summed in j order
 *                      (+ Down_s(SiLU(Gate_s x_t) * (Up_s x_t)) with weight 1
 *                       when a shared expert is configured)
 *
 * Weight format (per expert, row-major, all device memory):
 *   w13  uint8  [E, 2I, H/2]   gate rows 0..I-1, up rows I..2I-1; byte j of a
 *                              row holds input 2j (low nibble) and 2j+1 (high
 *                              nibble); code c in 0..15 means (c - 8) * scale
 *   s13  fp16   [E, 2I, H/32]  one scale per 32 consecutive inputs of a row
 *   w2   uint8  [E, H, I/2]    down projection, same packing along I
 *   s2   fp16   [E, H, I/32]
 * Activations x: bf16 [M, H]; router logits: fp32 [M, E]; out: bf16 [M, H].
 * All row-major and contiguous.
 *
 * Arithmetic and ranges: each token's hidden row is scaled by a power of two
 * 2^-e chosen from its largest |x| (2^e <= max|x_t| < 2^(e+1), e clamped to
 * [-60, 60]) and converted to fp16; the scaling is exact, so any finite bf16
 * row with max|x_t| in [2^-60, 2^61) enters the products with fp16 rounding
 * only below 2^-14 of its largest value.  h = SiLU(gate)*up is held in fp16
 * times 2^-2e, so |h_t| must stay below 65504 * 4^e (and is rounded to fp16
 * subnormals below 2^-14 * 4^e); an overflow gives inf/NaN in that token's
 * output.  The MFMA tiles hold decoded weights at odd input offsets times 16
 * in fp16, so group scales must not exceed 511.75 (16*8*s <= 65504); scales
 * are otherwise any finite fp16, subnormals included.  Logits must be finite.
 * Which kernel a call uses depends on the average number of routed rows per
 * expert, M*top_k/E:
 *   <= 1.75   dot-product GEMV on items of <= 2 rows: per 32-input group,
 *             sum(x*c) in fp32 (exact products) minus 8*sum(x), times the
 *             group's scale in fp32 (an all-8 group is zero only up to
 *             fp32 cancellation); a launch of fewer than 128 blocks splits
 *             K over up to one block per 512 inputs, and the last block of
 *             each split set adds the fp32 partial sums in split order;
 *   > 1.75    128-row MFMA tiles: codes decoded to fp16 operands
 *             ((c-8)*scale rounded to nearest even), products accumulated
 *             in fp32 by MFMA.
 * The weighted per-slot results are rounded to bf16 (nearest even) in the
 * workspace, summed per token in fp32 in slot order, and out is rounded to
 * bf16 (nearest even).  Results are deterministic for a given M (the regime,
 * the work items and the K splits depend on M, so a token's result may
 * differ in its last bits between calls of different M).
 *
 * Ownership: the caller owns every buffer.  The layer handle borrows the
 * weight pointers (and the expert bias) for its lifetime: the dot-product
 * GEMV reads the codes and scales as given.  It also copies the codes and
 * scales once, at creation, into one device allocation it owns (the same
 * size as the weights, freed by qmoe_layer_destroy) in the order the MFMA
 * tiles' loads read them.  So the weights must not change while the handle
 * lives: after new weights are written, destroy the handle and create a new
 * one (a handle that saw the change would compute decode-sized calls with
 * the new weights and tile calls with the old).  Forward calls allocate
 * nothing: per-call scratch lives in a caller-provided workspace whose size
 * comes from qmoe_workspace_size().
 *
 * Streams: every enqueueing call takes a hipStream_t (as void*, NULL = the
 * default stream), only enqueues work on it and never synchronises.  Faults
 * inside kernels surface at the caller's next synchronisation.
 *
 * Errors: calls return QMOE_OK (0) or a negative status; the message of the
 * last failure on the calling thread is returned by qmoe_last_error().  No
 * call falls back to another implementation: an unsupported case is an
 * error.  Argument checks run before any device query, so they work
 * without a GPU.
 *
 * Thread safety: a handle may be used from several threads only if each
 * thread uses its own workspace; the statistics counters are atomic.
 */
#ifndef QMOE_H
#define QMOE_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define QMOE_VERSION 4

enum qmoe_status {
  QMOE_OK = 0,
  QMOE_ERR_ARG = -1,          /* a null pointer, a bad size, a bad index */
  QMOE_ERR_UNSUPPORTED = -2,  /* a shape or device this build does not run */
  QMOE_ERR_WORKSPACE = -3,    /* workspace missing or smaller than required */
  QMOE_ERR_DEVICE = -4,       /* a HIP runtime query failed (e.g. no GPU) */
  QMOE_ERR_LAUNCH = -5        /* a kernel launch or async copy failed */
};

/* Limits of this build. */
#define QMOE_MAX_EXPERTS 1024
#define QMOE_MAX_TOPK 32
#define QMOE_GROUP 32

typedef struct {
  int32_t E;          /* routed experts, 1..QMOE_MAX_EXPERTS */
  int32_t H;          /* hidden size, multiple of 128 */
  int32_t I;          /* intermediate size, multiple of 128 */
  int32_t top_k;      /* 1..min(E, QMOE_MAX_TOPK) */
  int32_t group_size; /* must be 32 */
  int32_t max_rows;   /* largest M a forward call may pass (>= 1) */
  const uint8_t* w13;
  const uint16_t* s13; /* fp16 bit patterns */
  const uint8_t* w2;
  const uint16_t* s2;
  /* Optional shared expert, applied to every token with weight 1.0: either
     all four NULL (none) or all four set; shapes as one routed expert. */
  const uint8_t* shared_w13;
  const uint16_t* shared_s13;
  const uint8_t* shared_w2;
  const uint16_t* shared_s2;
  /* Expert-parallel shard ("The MoE Throughput Lever ...", section "The
     Architectural Implication: Refining the Engine Design": experts sharded
     over GPUs): the handle holds and computes only experts local_first ..
     local_first + local_count - 1 of the E it routes over; w13/s13/w2/s2
     then hold local_count experts (local expert 0 = expert local_first).
     Routing ranks all E logits; slots routed to other experts are skipped,
     so out is this shard's partial sum over the token's local slots (plus
     the shared expert, if configured); the shards' outputs add up to the
     whole layer's.  local_count = 0: all E experts are local. */
  int32_t local_first;
  int32_t local_count;
  /* Router scoring.  The pages state top-8 routing over 384 experts but not
     how the experts are scored ("The MoE Throughput Lever ...", section "The
     Context: Why This Measurement Matters").
     QMOE_SCORING_SOFTMAX (0, the default): the top_k logits, weights = the
     softmax over all E logits renormalised over the selected experts.
     QMOE_SCORING_SIGMOID (1): the sigmoid router of the model family whose
     shapes the pages benchmark: each expert's score s = 1/(1+e^-l) in fp32;
     the top_k by the fp32 key s + expert_bias[e] (ties to the lower index;
     the bias steers selection only); weights = s / (sum of the selected s) *
     routed_scale.  expert_bias: NULL (no bias) or device fp32 [E] over all E
     experts (also for a shard), borrowed like the weights and read by every
     routing call; only with the sigmoid scoring.  Its values must be finite
     (it is not read at creation; a non-finite bias leaves the selection
     undefined).  routed_scale: 0 means 1; otherwise finite and > 0
     (QMOE_ERR_ARG otherwise). */
  int32_t scoring;
  float routed_scale;
  const float* expert_bias;
} qmoe_layer_desc;
#define QMOE_SCORING_SOFTMAX 0
#define QMOE_SCORING_SIGMOID 1

typedef struct qmoe_layer qmoe_layer;

/* Validate the description and create a handle.  Fails with QMOE_ERR_ARG on
   a bad field (the message names it), then with QMOE_ERR_DEVICE if no HIP
   device can be queried and QMOE_ERR_UNSUPPORTED if the current device is
   not gfx950.  Then copies the weight codes and scales (w13, s13, w2, s2
   and the shared expert's; all of them at their full sizes, also for a
   handle used only for router calls) into the handle's own device
   allocation in tile order, for the MFMA tiles: each 16-row block's codes
   stored 128 inputs at a time (64 bytes of each of its rows, 1 KiB), the
   16 bytes of row r at bytes 16 kq .. 16 kq + 15 of that span placed at
   16 (16 kq + r), and its scales 512 inputs at a time (16 groups of each
   row, 512 bytes), the scales of groups 4 kq .. 4 kq + 3 of row r placed at
   8 (16 kq + r), so each MFMA-tile load instruction reads 1 KiB or 512
   bytes contiguous.  The device is synchronised before the copy (the
   weights must have been written, on any stream) and after it;
   QMOE_ERR_DEVICE if the allocation fails.  The scales' values are not
   checked: the ranges above (group scales <= 511.75) are the caller's to
   keep.  Nothing is read from the environment. */
int qmoe_layer_create(const qmoe_layer_desc* desc, qmoe_layer** out);
void qmoe_layer_destroy(qmoe_layer* layer);

/* Bytes of workspace a call with M tokens needs (0 <= M <= max_rows): one
   scratch allocation per call holds routing, work list, h, y and split-K
   partials (the single scratch allocation the engagement receipts of
   "perf(exl3): accelerate fat-expert prefill" count, section "Engagement
   and fallback proof").  The caller allocates and owns it. */
int qmoe_workspace_size(const qmoe_layer* layer, int64_t M, size_t* bytes);

/* Enqueue a clear of a workspace's control words.  Optional: no call
   depends on what a workspace held before. */
int qmoe_workspace_init(qmoe_layer* layer, void* workspace, size_t ws_bytes, void* stream);

/* The whole layer ("The MoE Throughput Lever ...", sections "The Context:
   Why This Measurement Matters" and "The Benchmark: What Was Measured"):
   route, gate+up, down, combine: four kernel launches,
   five for calls of more than 64 tokens (their routing takes two: the top-k
   of every token, then one block per 64-token chunk for the counts, the
   scan, the sorted positions and the work list), and two more in a mixed
   call (QMOE_REGIME_MIXED: gate+up and down each also run the dot-product
   GEMV over the experts of 1-2 rows).
   x: bf16 [M,H] (any finite values; see the ranges above); logits: fp32
   [M,E], finite; out: bf16 [M,H] (device pointers, 16-byte aligned).
   M == 0 is a no-op.  Graph-capturable for a fixed M (no memset nodes). */
int qmoe_forward(qmoe_layer* layer, const void* x, const float* logits, int64_t M,
                 void* out, void* workspace, size_t ws_bytes, void* stream);

/* For callers that cannot allocate device memory (code under HIP graph
   capture, serving loops or harnesses that forbid allocation): the whole
   layer exactly as qmoe_forward (same kernels, same results), with its
   scratch in a device array the library holds for each GPU
   (QMOE_STATIC_SCRATCH_BYTES, held until the process ends) instead of a
   caller workspace.  Allocates nothing.  The caller still passes x, logits
   and out.  A call whose workspace (qmoe_workspace_size) would exceed the
   array returns QMOE_ERR_WORKSPACE without enqueueing anything (the
   384-expert, H=7168, I=2048, top-8 layer fits up to about 190 tokens).
   Every call on one GPU, from any layer, uses that GPU's one array: calls
   that overlap on a GPU (different streams or threads) race, and the caller
   must serialise them.  Routing and intermediates of such a call are not
   readable through qmoe_read_routing / qmoe_read_intermediate. */
#define QMOE_STATIC_SCRATCH_BYTES (32u << 20)
int qmoe_forward_static(qmoe_layer* layer, const void* x, const float* logits, int64_t M, void* out,
                        void* stream);

/* The router in front of the layer ("The MoE Throughput Lever: Quantifying
   the INT4 Marlin GEMM on Blackwell PRO 6000", section "The Context: Why
   This Measurement Matters" states top-8 routing over 384 experts, not how
   the scores are made; this build reads it as a linear map):
     logits[t, e] = sum_k x[t, k] * w_router[e, k]
   x: bf16 [M,H]; w_router: bf16 [E,H], row-major (device pointers, 16-byte
   aligned); logits: fp32 [M,E] (device).  Products of two bf16 values are
   exact in fp32; the sum is accumulated in fp32 (bf16 MFMA above 16 tokens,
   fp32 FMAs below).  One kernel launch; M == 0 is a no-op. */
int qmoe_router_logits(qmoe_layer* layer, const void* x, const void* w_router, int64_t M, float* logits,
                       void* stream);

/* The router and the whole layer in one call: qmoe_router_logits into the
   workspace (its size already covers the M*E logits), then qmoe_forward on
   them.  Same arguments as qmoe_forward with w_router in place of logits. */
int qmoe_forward_router(qmoe_layer* layer, const void* x, const void* w_router, int64_t M, void* out,
                        void* workspace, size_t ws_bytes, void* stream);

/* The same four steps one at a time, on one workspace and in this order
   (each reads what the previous one left in the workspace).  They let a
   caller time or check each step alone.  Sources: top-8 routing ("The MoE
   Throughput Lever ...", section "The Context: Why This Measurement
   Matters"); the per-expert counts and their scan ("Detailed results",
   section "Nsight Compute on the stock kernel"); sorted routing, the
   stacked gate+up GEMM over a shared input and the results scattered back
   per token ("perf(exl3): accelerate fat-expert prefill", description and
   sections "Rollout" and "Engagement and fallback proof": its direct and
   scatter calls); INT4 group-32 weights with 16-bit activations ("The MoE
   Throughput Lever ...", section "The Benchmark: What Was Measured").
   Errors: as qmoe_forward (argument, workspace and device checks return
   before anything is enqueued).
     qmoe_route     top-k routing, expert counts and their exclusive scan,
                    the stable sort of routed slots by expert, the flat list
                    of (expert, row-tile) work items, and x converted to the
                    GEMM operand format;
     qmoe_gate_up   per expert, the stacked gate+up product with
                    h = SiLU(gate)*up;
     qmoe_down      per expert, the down product times the routing weight,
                    written per (token, slot);
     qmoe_combine   out[t] = sum over slots j (in order) + shared expert. */
int qmoe_route(qmoe_layer* layer, const void* x, const float* logits, int64_t M,
               void* workspace, size_t ws_bytes, void* stream);
int qmoe_gate_up(qmoe_layer* layer, int64_t M, void* workspace, size_t ws_bytes, void* stream);
int qmoe_down(qmoe_layer* layer, int64_t M, void* workspace, size_t ws_bytes, void* stream);
int qmoe_combine(qmoe_layer* layer, int64_t M, void* out, void* workspace, size_t ws_bytes,
                 void* stream);

/* Copy the routing results of the last qmoe_route/qmoe_forward on this
   workspace into caller buffers (device pointers; any may be NULL):
   ids int32 [M,k], w fp32 [M,k], counts int32 [L], offsets int32 [L+1],
   perm int32 [M*k] (perm[pos] = t*k+j, experts in order, tokens ascending
   within an expert), L = the local experts (E unless the layer is an
   expert-parallel shard; then only the first offsets[L] entries of perm are
   this shard's). */
int qmoe_read_routing(qmoe_layer* layer, int64_t M, const void* workspace, size_t ws_bytes,
                      int32_t* ids, float* w, int32_t* counts, int32_t* offsets,
                      int32_t* perm, void* stream);

/* Copy an intermediate of the last call into fp32 rows in slot order
   (h is held as fp16, y as bf16; both convert to fp32 exactly)
   (row t*k+j for routed slot j of token t; rows M*k+t for the shared expert):
   which = 0: h = SiLU(gate)*up, [M*k (+M), I]  (after qmoe_gate_up)
   which = 1: y = w * Down(h),   [M*k (+M), H]  (after qmoe_down) */
int qmoe_read_intermediate(qmoe_layer* layer, int64_t M, const void* workspace, size_t ws_bytes,
                           int32_t which, float* out_f32, void* stream);

/* Decode one expert's weights with the same device function the GEMMs use,
   from the handle's tile-order copy of the codes and scales (so the copy
   is checked too), and write the fp16 operand values in natural order: which = 0:
   [2I, H] from w13/s13, which = 1: [H, I] from w2/s2.  expert == E selects
   the shared expert.  out: uint16 fp16 bit patterns, device memory. */
int qmoe_dequant_debug(qmoe_layer* layer, int32_t expert, int32_t which, uint16_t* out_f16,
                       void* stream);

/* Host-side counters, bumped by the enqueueing calls (no device readback). */
typedef struct {
  uint64_t forward_calls;
  uint64_t route_calls;       /* qmoe_route, also inside qmoe_forward */
  uint64_t gemm_launches;     /* gate+up and down kernel launches */
  uint64_t launches;          /* every kernel launch */
  uint64_t workspace_inits;   /* qmoe_workspace_init calls */
  uint64_t workspace_bytes_last;
  uint64_t workspace_bytes_peak;
  uint64_t prefill_tiles;     /* gate+up launches on 128-row MFMA tiles */
  uint64_t gemv_tiles;        /* gate+up launches on <= 2-row dot-product items
                                 (a mixed call counts one of each) */
  uint64_t gemv_nt_launches;  /* dot-product launches (gate+up and down) reading the
                                 weight codes with the non-temporal cache policy:
                                 calls with M*top_k <= E and no shared expert */
  uint64_t splitk_launches;   /* dot-product launches with K split over blocks */
} qmoe_stats;

int qmoe_get_stats(const qmoe_layer* layer, qmoe_stats* out);
int qmoe_reset_stats(qmoe_layer* layer);

/* Per-call engagement receipt: what the last completed forward call on the
   handle (qmoe_forward or qmoe_forward_static) enqueued, recorded on the
   host as it enqueued it (no device readback), so a caller can prove which
   kernels ran and that nothing fell back.  The counterpart of the per-call
   tier and engagement counters in "perf(exl3): accelerate fat-expert
   prefill", sections "Summary" and "Engagement and fallback proof". */
#define QMOE_REGIME_GEMV 1   /* dot-product GEMV on work items of <= 2 routed rows */
#define QMOE_REGIME_TILES 2  /* 128-row MFMA tiles */
#define QMOE_REGIME_MIXED 3  /* tiles for the experts of more than 2 rows and the
                                dot-product GEMV (one more launch per product) for
                                those of 1-2 rows: tile-regime calls that average
                                at most 4 routed rows per expert */
typedef struct {
  uint64_t seq;             /* 1-based number of the forward call on this handle */
  int64_t M;
  int32_t regime;           /* QMOE_REGIME_GEMV, _TILES or _MIXED */
  int32_t rows_per_item;    /* routed rows per work item: 2 or 128 */
  int32_t nt_codes;         /* 1: the GEMV read weight codes non-temporal */
  int32_t shared_expert;    /* 1: a shared expert was applied */
  int32_t launches;         /* kernel launches the call enqueued */
  int32_t route_kernels;    /* 1 (calls of <= 64 tokens) or 2 */
  int64_t max_items;        /* work items the GEMM grids were sized for (an upper
                               bound of the items routing builds) */
  int64_t gate_up_blocks;   /* grid sizes of the launches (a mixed call: of its
                               tile launches; its dot-product launches have
                               local experts x column blocks) */
  int64_t down_blocks;
  int64_t combine_blocks;
  uint64_t workspace_bytes; /* workspace bytes the call used */
  int32_t static_scratch;   /* 1: qmoe_forward_static (library scratch) */
  int32_t router;           /* 1: qmoe_forward_router (logits computed in the call) */
  int32_t splits_gate_up;   /* K splits of the dot-product launches (1 = none) */
  int32_t splits_down;
} qmoe_receipt;

/* Copy the receipt of the last completed forward call (QMOE_ERR_ARG if none
   has completed). */
int qmoe_last_receipt(const qmoe_layer* layer, qmoe_receipt* out);

/* Enqueue a device-to-device copy of the number of work items the last
   routing on this workspace built (int32, device memory): the items the GEMM
   grids actually processed, sum over experts of ceil(count / rows_per_item)
   plus the shared expert's. */
int qmoe_read_item_count(qmoe_layer* layer, int64_t M, const void* workspace, size_t ws_bytes,
                         int32_t* n_items, void* stream);

/* Message of the last failing call on this thread ("" if none). */
const char* qmoe_last_error(void);
int qmoe_version(void);

#ifdef __cplusplus
}
#endif
#endif /* QMOE_H */
