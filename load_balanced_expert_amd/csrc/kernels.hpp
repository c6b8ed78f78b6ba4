// Internal launchers of libmoe (host side, C++ linkage).  Arguments are
// validated by the C-ABI layer before any of these is called.
#pragma once
#include <hip/hip_runtime.h>

#include "prefix.hpp"
#include <stddef.h>
#include <stdint.h>

namespace moe {

// ---------------------------------------------------------------- router
struct RoutePlan {
  bool fused;      // logits tile kept in LDS (n <= kFusedMaxN)
  bool mfma;       // bf16 x on matrix cores (exact 3-way bf16 split of W_r)
  int npad;        // experts padded (fused: multiple of 32, else of 128)
  int dpad;        // d padded to a multiple of 32 (mfma)
  size_t planes_bytes;
  size_t logits_bytes;
  int kg;          // fused route: workgroups (K ranges) per 32-token tile
  size_t kpart_bytes;   // kg > 1: per-K-group logit tiles
};
constexpr int kFusedMaxN = 256;
RoutePlan route_plan(int64_t m, int d, int n, bool x_bf16);

struct RouteArgs {
  const void* x;
  int64_t m;
  int d, n, npad, dpad, k;
  int score;       // 0 softmax, 1 sigmoid
  int gate;        // 0 prob, 1 renorm
  int x_bf16;      // storage dtype of x
  const float* w_r;
  const float* bias;
  const uint16_t* planes;
  bool planes_ready;  // planes already hold the split of w_r
  bool parts_apart;   // set by launch_route: partial tiles after the x tile
  float* logits;   // big-n path only
  int32_t* idx;
  float* gate_out;
  int32_t* counts;
  float* prob_sum;     // optional
  float* f;            // optional load statistics
  float* P;
  float* aux;
  float alpha;
  uint64_t* chunks;       // [route workgroups, n] packed (count, score sum) chunk rows (workspace)
  bool want_psum;         // score sums wanted (prob_sum, P or aux)
  int sup;                // chunks per super chunk
  int32_t capacity;       // < 0: no capacity prefix sums
  int32_t* expert_offsets;
  int32_t* expert_rows;   // [n] kept rows per expert, or nullptr
  bool padded;            // capacity-padded layout
  int32_t* super_prefix;
  uint32_t* done;         // completion ticket (control region)
  int lds_region_ints;    // set by launch_route
  bool finish;            // false: store the chunk rows only (the dispatch finishes)
  int kg;                         // workgroups per token tile (RoutePlan::kg)
  int rows_sub;                   // big-n epilogue: tokens per LDS sub-tile (set by launch_route)
  float* kpart;                   // kg > 1: [tiles][kg][32][npad] partial logits (workspace)
  uint32_t* tile_tickets;         // kg > 1: [tiles] (control region)
  int32_t* sup_counts;            // finish == false or fin_super: per-super-chunk sums (atomics)
  unsigned long long* sup_psum;
  bool fin_super;                 // finish from the per-super-chunk sums (n <= 256), not the chunk rows
  // the Loss-Free step done by the finish (stand-alone route only; all optional)
  int64_t* gcounts;               // [n] global-batch counts += counts
  int64_t* gtokens;               // [1] global-batch tokens += m
  float* lf_bias;                 // [n] the bias, updated in place after it was used to route
  float gamma;
};
hipError_t launch_route(const RoutePlan& plan, const RouteArgs& a, hipStream_t s);
int route_chunk_tokens(const RoutePlan& plan);  // tokens per route workgroup (= dispatch chunk)
// whether the route kernel reads W_r directly (no prepared planes needed)
bool route_direct(const RoutePlan& plan, int d, int n);
hipError_t launch_router_prepare(const RoutePlan& plan, int d, int n, const float* w_r, uint16_t* planes,
                                 hipStream_t s);

// ---------------------------------------------------------------- stats
hipError_t launch_stats(int64_t m, int n, int k, const int32_t* counts, const float* prob_sum,
                        float alpha, float* f, float* P, float* aux, int64_t* gcounts,
                        int64_t* gtokens, float* bias, float gamma, hipStream_t s);
hipError_t launch_global_aux(int n, const int64_t* gcounts, const int64_t* gtokens, const float* P,
                             int nb, float alpha, float* fg, float* losses, float* loss_mean,
                             const float* micro_aux, float global_weight, float micro_weight, float* hybrid,
                             float* hybrid_mean, hipStream_t s);

// ---------------------------------------------------------------- dispatch
struct DispatchArgs {
  const int32_t* idx;
  int64_t pairs;        // m * k
  int k, n, nbits;
  int32_t capacity;     // >= 0 (unlimited is passed as pairs)
  int chunk_tokens;     // tokens per chunk (== route workgroup tokens when the route made the counts)
  int nch, sup;         // chunks, chunks per super chunk
  uint64_t* chunks;       // [nch, n] packed chunk rows (count in the low word)
  int32_t* super_prefix;  // [ceil(nch / sup), n]
  int32_t* token_to_row;
  uint8_t* drop_mask;
  int32_t* expert_offsets;
  int32_t* expert_rows;   // [n] kept rows per expert, or nullptr
  bool padded;            // capacity-padded layout: expert j owns rows [j C, (j + 1) C)
  int32_t* row_to_token;
  const void* x;
  void* dispatched;
  int64_t row_bytes;    // d * element size
  uint32_t* done;       // completion ticket (control region)
  // self_prefix: the route kernel left only its chunk count rows and the
  // per-super-chunk sums; every dispatch workgroup derives the expert totals,
  // its chunk bases and the offsets, and workgroup 0 publishes the load
  // statistics (nullptr: not wanted)
  bool self_prefix;
  const int32_t* sup_counts;            // [nsup][n] (control region)
  const unsigned long long* sup_psum;   // [nsup][n] fixed point, 2^-32
  int32_t* counts;
  float* prob_sum;
  float* f;
  float* P;
  float* aux;
  float alpha;
  // self_prefix, workgroup 0: global-batch accumulation and the Loss-Free bias
  // update from the expert totals (nullptr: not wanted)
  int64_t* gcounts;
  int64_t* gtokens;
  float* lf_bias;
  float gamma;
};
constexpr int kDispMaxChunkPairs = 4096;
// chunk tokens for m tokens x k choices given the route workgroup size
inline int dispatch_chunk_tokens(int route_tokens, int k) {
  return route_tokens * k <= kDispMaxChunkPairs ? route_tokens : (kDispMaxChunkPairs / k > 0 ? kDispMaxChunkPairs / k : 1);
}
size_t dispatch_ws_bytes(int64_t m, int k, int n, int chunk_tokens);
hipError_t launch_dispatch(const DispatchArgs& a, bool prefix_ready, hipStream_t s);
// whether the dispatch can derive the prefix from nch chunk rows of n experts
bool dispatch_self_prefix_ok(int nch, int n);

// ---------------------------------------------------------------- expert FFN
size_t ffn_ws_bytes(int64_t rows_bound, int d_ff);
// rows (nullable): rows of expert j = rows[j] from offsets[j] (capacity-padded
// layout); else offsets[j + 1] - offsets[j]
// packed: w1 and w2 hold moe_expert_weights_pack's layout (only where ffn_packed_ok)
hipError_t launch_expert_ffn(int n, int d, int d_ff, int rows_max, const int32_t* offsets, const int32_t* rows,
                             const uint16_t* D, const uint16_t* w1, const uint16_t* w2,
                             uint16_t* hidden, uint16_t* y, hipStream_t s, bool packed = false);
// whether both GEMMs of the FFN run on the weight-stream kernel, the only one that reads packed weights
bool ffn_packed_ok(int d, int d_ff, int rows_max, int n);
// [n][N][K] bf16 weights -> the stream kernel's fragment order (N % 32 == 0, K % 64 == 0)
hipError_t launch_pack_weights(int64_t n, int N, int K, const uint16_t* w, uint16_t* p, hipStream_t s);

// ---------------------------------------------------------------- combine
// clear (optional): bytes of device memory the first workgroup zeroes (16-byte multiple)
hipError_t launch_combine(int64_t m, int d, int k, const void* y, bool y_bf16, const float* gate,
                          const int32_t* token_to_row, const void* residual, void* out,
                          bool x_bf16, hipStream_t s, void* clear = nullptr, size_t clear_bytes = 0);

// ---------------------------------------------------------------- balanced assignment
size_t balance_ws_bytes(int64_t m, int n, int k, bool exact);
// whether the exact completion handles these sizes (n <= 64, or n <= 128 within its LDS budget)
bool exact_completion_supported(int64_t m, int n, int k);
struct BalanceArgs {
  int64_t m;
  int n, k;
  int64_t q;
  const float* s;
  float* beta;
  int iters, mode, exact;
  // quantile form (the demo code's 1 - k/n quantile with linear interpolation):
  // the lower order statistic's 0-based descending rank and the weight of the
  // next larger one, per axis (set by launch_balance); bip clips α and β at 0
  bool quantile, bip;
  int rank_row;
  float g_row;
  int64_t rank_col;
  float g_col;
  int32_t* idx;
  int32_t* counts;
  float* alpha_out;
  int32_t* info;
  void* ws;          // after the control words
  uint32_t* done;    // completion ticket (control region)
  // mini-batch duals: the tokens fall into blocks of beta_rows consecutive rows,
  // each with its own β row (row kernels: β block i / beta_rows; column kernel:
  // one segment of beta_rows keys per block).  One block: beta_rows = m.
  int64_t beta_rows;
  int nblocks;
};
hipError_t launch_balance(const BalanceArgs& a, hipStream_t s);
// mini-batch β: QB steps on every block of batch_rows tokens at once, the
// blocks' β averaged (fp64, block order) into a.beta
hipError_t launch_balance_minibatch(const BalanceArgs& a, hipStream_t s);
// SignSGD steps on β (n <= 256), then the counting top-k of the final β
hipError_t launch_signsgd(const BalanceArgs& a, float gamma, hipStream_t s);

// ---------------------------------------------------------------- backward
struct BackwardArgs {
  int64_t m;
  int d, n, k, d_ff;
  int64_t rows_bound;   // rows of the dispatched buffer
  int rows_max;         // most rows any expert holds
  bool x_bf16;
  float alpha;
  const void* x;
  const float* w_r;
  const uint16_t* w1;
  const uint16_t* w2;
  const int32_t* idx;
  const float* gate;
  const int32_t* counts;
  const int32_t* t2r;
  const int32_t* offsets;
  const int32_t* rows;   // rows per expert (capacity layout) or nullptr (compact offsets)
  const uint16_t* dispatched;
  const uint16_t* hidden;
  const uint16_t* y;
  const float* dout;
  float* dx;
  float* dw_r;
  float* dw1;
  float* dw2;
  void* ws;
};
size_t backward_ws_bytes(int64_t m, int d, int n, int k, int64_t rows_bound, int d_ff);
hipError_t launch_backward(const BackwardArgs& b, hipStream_t s);

}  // namespace moe
