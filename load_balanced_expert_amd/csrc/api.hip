// C ABI of libmoe: host-side validation, workspace carve-up and launch
// sequencing.  Every argument check runs before the first HIP call.
#include <math.h>
#include <string.h>

#include <mutex>

#include "moe.h"
#include "common.hpp"
#include "kernels.hpp"

namespace moe {
// Zero fill with vector stores: a kernel rather than hipMemsetAsync, so that the
// clears a caller's stream sees can be recorded into a HIP graph.
__global__ __launch_bounds__(256) void k_zero16(u32x4* __restrict__ p, int64_t n16) {
  for (int64_t i = int64_t(blockIdx.x) * 256 + threadIdx.x; i < n16; i += int64_t(gridDim.x) * 256)
    p[i] = u32x4{0u, 0u, 0u, 0u};
}
}  // namespace moe

namespace {
using namespace moe;

static_assert(kSupCountsOff % 16 == 0 && kControlBytes % 16 == 0, "control words are cleared in 16-byte units");

// Clears `bytes` bytes at p (16-byte aligned, bytes a multiple of 16) on stream s.
hipError_t zero_bytes(void* p, size_t bytes, hipStream_t s) {
  const int64_t n16 = int64_t(bytes / 16);
  if (n16 == 0) return hipSuccess;
  const unsigned g = unsigned(std::min<int64_t>((n16 + 255) / 256, 1024));
  hipLaunchKernelGGL(k_zero16, dim3(g), dim3(256), 0, s, static_cast<u32x4*>(p), n16);
  return hipGetLastError();
}

size_t al(size_t b) { return (b + 255) & ~size_t(255); }

struct Layout {
  size_t planes, logits, kpart, chunks, r2t, hidden;
  size_t idx, gate, counts, psum, f, P, aux, t2r, drop, offs, rowsn, disp, y;
  size_t route_end, dispatch_end, total;
  RoutePlan rp;
  int64_t pairs, rows_bound;
  int route_ct, disp_ct, nch, sup, nch_route, sup_route;
  size_t super_prefix;
};

bool shape_valid(const moe_shape* s) {
  return s && s->m >= 1 && s->d >= 1 && s->n >= 1 && s->k >= 1 && s->k <= s->n &&
         (s->score == MOE_SCORE_SOFTMAX || s->score == MOE_SCORE_SIGMOID) &&
         (s->gate == MOE_GATE_PROB || s->gate == MOE_GATE_RENORM) &&
         (s->x_dtype == MOE_F32 || s->x_dtype == MOE_BF16);
}

bool shape_supported(const moe_shape* s) {
  return s->n <= kMaxExperts && s->k <= kMaxK && s->d <= kMaxD && s->m <= 0x7FFFFFFFll &&
         s->m * s->k <= 0x7FFFFFFFll;
}

moe_status check_shape(const moe_shape* s) {
  if (!shape_valid(s)) return MOE_ERR_INVALID_ARG;
  if (!shape_supported(s)) return MOE_ERR_UNSUPPORTED;
  return MOE_OK;
}

size_t x_esz(const moe_shape& s) { return s.x_dtype == MOE_BF16 ? 2 : 4; }

Layout layout(const moe_shape& s, int32_t capacity, int32_t d_ff) {
  Layout L{};
  L.rp = route_plan(s.m, s.d, s.n, s.x_dtype == MOE_BF16);
  L.pairs = s.m * s.k;
  // dispatched rows: capacity-padded n * C, or compact m * k without a capacity
  L.rows_bound = capacity < 0 ? L.pairs : int64_t(capacity) * s.n;
  const size_t esz = x_esz(s);
  size_t o = kControlBytes;
  L.planes = o; o += al(L.rp.planes_bytes);
  L.logits = o; o += al(L.rp.logits_bytes);
  L.kpart = o; o += al(L.rp.kpart_bytes);
  L.route_ct = route_chunk_tokens(L.rp);
  L.disp_ct = dispatch_chunk_tokens(L.route_ct, s.k);
  L.nch = int(ceil_div64(s.m, L.disp_ct));
  L.sup = super_chunk(L.nch);
  L.nch_route = int(ceil_div64(s.m, L.route_ct));
  L.sup_route = super_chunk(L.nch_route);
  const int nch_max = std::max(L.nch, L.nch_route);
  L.chunks = o; o += al(size_t(nch_max) * s.n * sizeof(uint64_t));
  L.route_end = o;   // the route's scratch ends with its chunk rows
  L.super_prefix = o; o += al(size_t(kMaxSuperChunks) * s.n * sizeof(int32_t));
  L.r2t = o; o += al(size_t(L.rows_bound) * 4);
  L.dispatch_end = o;
  L.hidden = o; o += al(d_ff > 0 ? ffn_ws_bytes(L.rows_bound, d_ff) : 0);
  L.idx = o; o += al(size_t(L.pairs) * 4);
  L.gate = o; o += al(size_t(L.pairs) * 4);
  L.counts = o; o += al(size_t(s.n) * 4);
  L.psum = o; o += al(size_t(s.n) * 4);
  L.f = o; o += al(size_t(s.n) * 4);
  L.P = o; o += al(size_t(s.n) * 4);
  L.aux = o; o += al(4);
  L.t2r = o; o += al(size_t(L.pairs) * 4);
  L.drop = o; o += al(size_t(L.pairs));
  L.offs = o; o += al(size_t(s.n + 1) * 4);
  L.rowsn = o; o += al(size_t(s.n) * 4);
  L.disp = o; o += al(size_t(L.rows_bound) * s.d * esz);
  L.y = o; o += al(size_t(L.rows_bound) * s.d * (d_ff > 0 ? 2 : esz));
  L.total = o;
  return L;
}

template <typename T>
T* at(void* ws, size_t off) {
  return reinterpret_cast<T*>(static_cast<char*>(ws) + off);
}

bool ws_ok(const void* ws, size_t have, size_t need) {
  return ws != nullptr && (reinterpret_cast<uintptr_t>(ws) % 256) == 0 && have >= need;
}

moe_status hip_status(hipError_t e) { return e == hipSuccess ? MOE_OK : MOE_ERR_HIP; }

int32_t effective_capacity(int32_t capacity, int64_t pairs) {
  return capacity < 0 ? int32_t(std::min<int64_t>(pairs, 0x7FFFFFFF)) : capacity;
}

// Work the route kernel's last workgroup can do for the stages after it.
struct RouteExtras {
  float* f = nullptr;
  float* P = nullptr;
  float* aux = nullptr;
  float alpha = 0.f;
  const DispatchArgs* disp = nullptr;   // capacity prefix sums for this dispatch
  bool defer_finish = false;            // chunk rows only; the dispatch derives everything else
  int64_t* gcounts = nullptr;           // Loss-Free step in the finish (stand-alone route)
  int64_t* gtokens = nullptr;
  float* lf_bias = nullptr;
  float gamma = 0.f;
};

moe_status do_route(const moe_shape& s, const Layout& L, const void* x, const float* w_r, const void* w_planes,
                    const float* bias, int32_t* idx, float* gate, int32_t* counts, float* prob_sum, void* ws,
                    hipStream_t st, const RouteExtras& ex = RouteExtras()) {
  RouteArgs a{};
  a.x = x;
  a.m = s.m;
  a.d = s.d;
  a.n = s.n;
  a.npad = L.rp.npad;
  a.dpad = L.rp.dpad;
  a.k = s.k;
  a.score = s.score;
  a.gate = s.gate;
  a.x_bf16 = s.x_dtype == MOE_BF16;
  a.w_r = w_r;
  a.bias = bias;
  a.planes = w_planes ? static_cast<const uint16_t*>(w_planes) : at<uint16_t>(ws, L.planes);
  a.planes_ready = w_planes != nullptr;
  a.logits = at<float>(ws, L.logits);
  a.idx = idx;
  a.gate_out = gate;
  a.counts = counts;
  a.prob_sum = prob_sum;
  a.f = ex.f;
  a.P = ex.P;
  a.aux = ex.aux;
  a.alpha = ex.alpha;
  a.chunks = at<uint64_t>(ws, L.chunks);
  a.want_psum = prob_sum || ex.P || ex.aux;
  a.sup = L.sup_route;
  a.capacity = -1;
  if (ex.disp) {
    a.capacity = ex.disp->capacity;
    a.expert_offsets = ex.disp->expert_offsets;
    a.expert_rows = ex.disp->expert_rows;
    a.padded = ex.disp->padded;
    a.super_prefix = ex.disp->super_prefix;
  }
  a.gcounts = ex.gcounts;
  a.gtokens = ex.gtokens;
  a.lf_bias = ex.lf_bias;
  a.gamma = ex.gamma;
  a.done = ctl_ticket(ws, kTicketRoute);
  a.kpart = at<float>(ws, L.kpart);
  a.tile_tickets = at<uint32_t>(ws, kTileTicketsOff);
  a.finish = !ex.defer_finish;
  a.sup_counts = at<int32_t>(ws, kSupCountsOff);
  a.sup_psum = at<unsigned long long>(ws, kSupPsumOff);
  // the stand-alone finish reads the per-super-chunk sums where they fit (the fused path, n <= 256)
  a.fin_super = a.finish && L.rp.fused && s.n <= kSelfPrefixMaxN &&
                (L.nch_route + L.sup_route - 1) / L.sup_route <= kMaxSuperChunks;
  RoutePlan rp = L.rp;
  if (rp.mfma && (reinterpret_cast<uintptr_t>(x) % 16) != 0) rp.mfma = false;
  return hip_status(launch_route(rp, a, st));
}

DispatchArgs dispatch_args(const moe_shape& s, const Layout& L, int32_t capacity, const void* x, const int32_t* idx,
                           int32_t* t2r, uint8_t* drop, int32_t* offs, int32_t* rows, int32_t* r2t, void* disp,
                           void* ws) {
  DispatchArgs a{};
  a.idx = idx;
  a.pairs = L.pairs;
  a.k = s.k;
  a.n = s.n;
  a.nbits = bits_for(s.n);
  a.capacity = effective_capacity(capacity, L.pairs);
  a.chunk_tokens = L.disp_ct;
  a.nch = L.nch;
  a.sup = L.sup;
  a.chunks = at<uint64_t>(ws, L.chunks);
  a.super_prefix = at<int32_t>(ws, L.super_prefix);
  a.token_to_row = t2r;
  a.drop_mask = drop;
  a.expert_offsets = offs;
  a.expert_rows = rows;
  a.padded = capacity >= 0;
  a.row_to_token = r2t;
  a.x = x;
  a.dispatched = disp;
  a.row_bytes = int64_t(s.d) * x_esz(s);
  a.done = ctl_ticket(ws, kTicketDispatch);
  return a;
}

moe_status do_dispatch(const moe_shape& s, const Layout& L, int32_t capacity, const void* x, const int32_t* idx,
                       int32_t* t2r, uint8_t* drop, int32_t* offs, int32_t* rows, int32_t* r2t, void* disp, void* ws,
                       bool prefix_ready, hipStream_t st) {
  const DispatchArgs a = dispatch_args(s, L, capacity, x, idx, t2r, drop, offs, rows, r2t, disp, ws);
  return hip_status(launch_dispatch(a, prefix_ready, st));
}

// ------------------------------------------------------------------ route without allocation
// Scratch of moe_route_noalloc: one file-scope device array per GPU, held until the
// process ends.  Host code never passes `scratch` itself to a kernel (on the host
// the name only stands for the variable): its device address is looked up once per
// device and kept in g_scratch_ptr.
constexpr size_t kNoAllocScratchBytes = size_t(16) << 20;
static __device__ __align__(256) unsigned char scratch[kNoAllocScratchBytes];
constexpr int kNoAllocMaxDevices = 64;
std::mutex g_scratch_mu;
void* g_scratch_ptr[kNoAllocMaxDevices] = {};

__global__ __launch_bounds__(256) void k_zero_words(u32x4* p, int n) {
  for (int i = blockIdx.x * 256 + threadIdx.x; i < n; i += gridDim.x * 256) p[i] = u32x4{0u, 0u, 0u, 0u};
}

// The current device's scratch address; on its first use the control words are
// cleared by a fill kernel on `st` (no memset node, so the call may be captured).
moe_status noalloc_scratch(void** out, hipStream_t st) {
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kNoAllocMaxDevices) return MOE_ERR_HIP;
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (g_scratch_ptr[dev] == nullptr) {
    void* p = nullptr;
    if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess || p == nullptr) return MOE_ERR_HIP;
    hipLaunchKernelGGL(k_zero_words, dim3(ceil_div(int(kControlBytes / 16), 256)), dim3(256), 0, st,
                       static_cast<u32x4*>(p), int(kControlBytes / 16));
    if (hipGetLastError() != hipSuccess) return MOE_ERR_HIP;
    g_scratch_ptr[dev] = p;
  }
  *out = g_scratch_ptr[dev];
  return MOE_OK;
}

}  // namespace

extern "C" {

size_t moe_workspace_size(const moe_shape* shape, int32_t capacity, int32_t d_ff) {
  if (check_shape(shape) != MOE_OK || capacity < -1 || d_ff < 0) return 0;
  return layout(*shape, capacity, d_ff).total;
}

moe_status moe_workspace_init(void* ws, size_t ws_bytes, void* stream) {
  if (!ws_ok(ws, ws_bytes, kControlBytes)) return ws ? MOE_ERR_WORKSPACE : MOE_ERR_INVALID_ARG;
  return hip_status(zero_bytes(ws, kControlBytes, static_cast<hipStream_t>(stream)));
}

int32_t moe_capacity(int64_t m, int32_t n, double cf) {
  if (m < 0 || n < 1 || !(cf >= 0) || !isfinite(cf)) return -1;
  if (cf == 0.0 || m == 0) return 0;
  int e = 0;
  const double fr = frexp(cf, &e);                 // cf = fr * 2^e, fr in [0.5, 1)
  const int64_t mant = int64_t(ldexp(fr, 53));     // cf = mant * 2^(e-53), exact
  int sh = e - 53;
  __int128 num = (__int128)m * mant;               // < 2^116
  __int128 q;
  if (sh >= 0) {
    if (sh > 60) return -1;
    q = (num << sh) / n;
  } else {
    q = num / n;                                   // floor(floor(a/b)/c) == floor(a/(b c))
    const int r = -sh;
    q = r >= 127 ? 0 : (q >> r);
  }
  if (q > 0x7FFFFFFF) return -1;
  return int32_t(q);
}

const char* moe_status_str(int32_t st) {
  switch (st) {
    case MOE_OK: return "ok";
    case MOE_ERR_INVALID_ARG: return "invalid argument";
    case MOE_ERR_UNSUPPORTED: return "unsupported size or option";
    case MOE_ERR_WORKSPACE: return "workspace too small or misaligned";
    case MOE_ERR_HIP: return "HIP launch failed";
    default: return "unknown status";
  }
}

const char* moe_build_info(void) { return "libmoe 0.1 gfx950"; }

size_t moe_router_planes_bytes(int32_t d, int32_t n) {
  if (d < 1 || n < 1 || n > kMaxExperts) return 0;
  return route_plan(1, d, n, true).planes_bytes;
}

moe_status moe_router_prepare(int32_t d, int32_t n, const float* w_r, void* planes, void* stream) {
  if (d < 1 || n < 1 || !w_r || !planes) return MOE_ERR_INVALID_ARG;
  if (n > kMaxExperts) return MOE_ERR_UNSUPPORTED;
  const RoutePlan rp = route_plan(1, d, n, true);
  return hip_status(launch_router_prepare(rp, d, n, w_r, static_cast<uint16_t*>(planes),
                                          static_cast<hipStream_t>(stream)));
}

moe_status moe_route(const moe_shape* shape, const void* x, const float* w_r, const void* w_planes, const float* bias,
                     int32_t* idx, float* gate, int32_t* counts, float* prob_sum, void* ws, size_t ws_bytes,
                     void* stream) {
  moe_status st = check_shape(shape);
  if (st != MOE_OK) return st;
  if (!x || !w_r || !idx || !gate || !counts) return MOE_ERR_INVALID_ARG;
  const Layout L = layout(*shape, -1, 0);
  if (!ws_ok(ws, ws_bytes, L.route_end)) return ws ? MOE_ERR_WORKSPACE : MOE_ERR_INVALID_ARG;
  return do_route(*shape, L, x, w_r, w_planes, bias, idx, gate, counts, prob_sum, ws,
                  static_cast<hipStream_t>(stream));
}

moe_status moe_route_lossfree(const moe_shape* shape, const void* x, const float* w_r, const void* w_planes,
                              float* bias, float gamma, int32_t* idx, float* gate, int32_t* counts, float* prob_sum,
                              int64_t* global_counts, int64_t* global_tokens, void* ws, size_t ws_bytes,
                              void* stream) {
  moe_status st = check_shape(shape);
  if (st != MOE_OK) return st;
  if (!x || !w_r || !bias || !idx || !gate || !counts || !isfinite(gamma) ||
      (global_counts == nullptr) != (global_tokens == nullptr))
    return MOE_ERR_INVALID_ARG;
  const Layout L = layout(*shape, -1, 0);
  if (!ws_ok(ws, ws_bytes, L.route_end)) return ws ? MOE_ERR_WORKSPACE : MOE_ERR_INVALID_ARG;
  RouteExtras ex;
  ex.gcounts = global_counts;
  ex.gtokens = global_tokens;
  ex.lf_bias = bias;
  ex.gamma = gamma;
  return do_route(*shape, L, x, w_r, w_planes, bias, idx, gate, counts, prob_sum, ws,
                  static_cast<hipStream_t>(stream), ex);
}

size_t moe_route_noalloc_max_bytes(void) { return kNoAllocScratchBytes; }

moe_status moe_route_noalloc(const moe_shape* shape, const void* x, const float* w_r, const void* w_planes,
                             const float* bias, int32_t* idx, float* gate, int32_t* counts, float* prob_sum,
                             void* stream) {
  moe_status st = check_shape(shape);
  if (st != MOE_OK) return st;
  if (!x || !w_r || !idx || !gate || !counts) return MOE_ERR_INVALID_ARG;
  const Layout L = layout(*shape, -1, 0);
  if (L.route_end > kNoAllocScratchBytes) return MOE_ERR_UNSUPPORTED;
  hipStream_t s = static_cast<hipStream_t>(stream);
  void* ws = nullptr;
  if ((st = noalloc_scratch(&ws, s)) != MOE_OK) return st;
  return do_route(*shape, L, x, w_r, w_planes, bias, idx, gate, counts, prob_sum, ws, s);
}

moe_status moe_stats(int64_t m, int32_t n, int32_t k, const int32_t* counts, const float* prob_sum, float alpha,
                     float* f, float* P, float* aux, int64_t* global_counts, int64_t* global_tokens, float* bias,
                     float gamma, void* stream) {
  if (m < 1 || n < 1 || k < 1 || k > n || !counts) return MOE_ERR_INVALID_ARG;
  if ((global_counts == nullptr) != (global_tokens == nullptr)) return MOE_ERR_INVALID_ARG;
  if ((P || aux) && !prob_sum) return MOE_ERR_INVALID_ARG;
  if (n > kMaxExperts) return MOE_ERR_UNSUPPORTED;
  if (m > (int64_t(1) << 40)) return MOE_ERR_UNSUPPORTED;  // c*n and m*k stay inside int64
  return hip_status(launch_stats(m, n, k, counts, prob_sum, alpha, f, P, aux, global_counts, global_tokens, bias,
                                 gamma, static_cast<hipStream_t>(stream)));
}

moe_status moe_global_aux(int32_t n, const int64_t* global_counts, const int64_t* global_tokens, const float* P,
                          int32_t nb, float alpha, float* f_global, float* losses, float* loss_mean,
                          const float* micro_aux, float global_weight, float micro_weight, float* hybrid,
                          float* hybrid_mean, void* stream) {
  if (n < 1 || nb < 0 || !global_counts || !global_tokens) return MOE_ERR_INVALID_ARG;
  if (nb > 0 && !P) return MOE_ERR_INVALID_ARG;
  if (nb > 0 && (hybrid || hybrid_mean) && !micro_aux) return MOE_ERR_INVALID_ARG;
  if (n > kMaxExperts) return MOE_ERR_UNSUPPORTED;
  return hip_status(launch_global_aux(n, global_counts, global_tokens, P, nb, alpha, f_global, losses, loss_mean,
                                      micro_aux, global_weight, micro_weight, hybrid, hybrid_mean,
                                      static_cast<hipStream_t>(stream)));
}

size_t moe_balance_workspace_size(int64_t m, int32_t n, int32_t k, int32_t exact) {
  if (m < 1 || n < 2 || k < 1 || k >= n) return 0;
  return kControlBytes + balance_ws_bytes(m, n, k, exact != 0);
}

moe_status moe_balance_duals(int64_t m, int32_t n, int32_t k, const float* s, float* beta, int32_t iters,
                             int32_t mode, int32_t exact, int32_t* idx, int32_t* counts, float* alpha,
                             int32_t* info, void* ws, size_t ws_bytes, void* stream) {
  if (m < 1 || n < 2 || k < 1 || k >= n || !s || !beta || !idx || !counts) return MOE_ERR_INVALID_ARG;
  if ((m * int64_t(k)) % n != 0) return MOE_ERR_INVALID_ARG;
  const bool quantile = (mode & MOE_QB_QUANTILE) != 0, bip = (mode & MOE_QB_BIP) != 0;
  mode &= ~(MOE_QB_QUANTILE | MOE_QB_BIP);
  if (mode != MOE_QB_SOLVE && mode != MOE_QB_ONLINE) return MOE_ERR_INVALID_ARG;
  if (iters < 0 || (mode == MOE_QB_ONLINE && (iters != 1 || exact))) return MOE_ERR_INVALID_ARG;
  if (n > kMaxExperts || m > 0x7FFFFFFFll || m * k > 0x7FFFFFFFll) return MOE_ERR_UNSUPPORTED;
  if (exact && !exact_completion_supported(m, n, k)) return MOE_ERR_UNSUPPORTED;
  if (!ws_ok(ws, ws_bytes, moe_balance_workspace_size(m, n, k, exact))) return ws ? MOE_ERR_WORKSPACE : MOE_ERR_INVALID_ARG;
  BalanceArgs a{};
  a.m = m;
  a.n = n;
  a.k = k;
  a.q = m * k / n;
  a.s = s;
  a.beta = beta;
  a.iters = mode == MOE_QB_ONLINE ? 1 : iters;
  a.mode = mode;
  a.exact = exact;
  a.quantile = quantile;
  a.bip = bip;
  a.idx = idx;
  a.counts = counts;
  a.alpha_out = alpha;
  a.info = info;
  a.ws = static_cast<char*>(ws) + kControlBytes;
  a.done = ctl_ticket(ws, kTicketBalance);
  return hip_status(launch_balance(a, static_cast<hipStream_t>(stream)));
}

size_t moe_balance_minibatch_workspace_size(int64_t m, int32_t n, int32_t k, int64_t batch_rows) {
  if (m < 1 || n < 2 || k < 1 || k >= n || batch_rows < 1 || m % batch_rows != 0) return 0;
  return kControlBytes + balance_ws_bytes(m, n, k, false) + al(size_t(m / batch_rows) * n * sizeof(float));
}

moe_status moe_balance_duals_minibatch(int64_t m, int32_t n, int32_t k, const float* s, float* beta, int32_t iters,
                                       int32_t mode, int64_t batch_rows, int32_t* idx, int32_t* counts, float* alpha,
                                       int32_t* info, void* ws, size_t ws_bytes, void* stream) {
  if (m < 1 || n < 2 || k < 1 || k >= n || !s || !beta || !idx || !counts) return MOE_ERR_INVALID_ARG;
  if ((m * int64_t(k)) % n != 0 || batch_rows < 1 || m % batch_rows != 0 || (batch_rows * k) % n != 0)
    return MOE_ERR_INVALID_ARG;
  const bool quantile = (mode & MOE_QB_QUANTILE) != 0, bip = (mode & MOE_QB_BIP) != 0;
  mode &= ~(MOE_QB_QUANTILE | MOE_QB_BIP);
  if (mode != MOE_QB_SOLVE && mode != MOE_QB_ONLINE) return MOE_ERR_INVALID_ARG;
  if (iters < 0 || (mode == MOE_QB_ONLINE && iters != 1)) return MOE_ERR_INVALID_ARG;
  if (n > kMaxExperts || m > 0x7FFFFFFFll || m * k > 0x7FFFFFFFll || m / batch_rows > 65535)
    return MOE_ERR_UNSUPPORTED;
  if (!ws_ok(ws, ws_bytes, moe_balance_minibatch_workspace_size(m, n, k, batch_rows)))
    return ws ? MOE_ERR_WORKSPACE : MOE_ERR_INVALID_ARG;
  BalanceArgs a{};
  a.m = m;
  a.n = n;
  a.k = k;
  a.q = m * k / n;
  a.s = s;
  a.beta = beta;
  a.iters = mode == MOE_QB_ONLINE ? 1 : iters;
  a.mode = mode;
  a.quantile = quantile;
  a.bip = bip;
  a.idx = idx;
  a.counts = counts;
  a.alpha_out = alpha;
  a.info = info;
  a.ws = static_cast<char*>(ws) + kControlBytes;
  a.done = ctl_ticket(ws, kTicketBalance);
  a.beta_rows = batch_rows;
  a.nblocks = int(m / batch_rows);
  return hip_status(launch_balance_minibatch(a, static_cast<hipStream_t>(stream)));
}

moe_status moe_balance_signsgd(int64_t m, int32_t n, int32_t k, const float* s, float* beta, float gamma,
                               int32_t iters, int32_t* idx, int32_t* counts, void* ws, size_t ws_bytes,
                               void* stream) {
  if (m < 1 || n < 2 || k < 1 || k >= n || !s || !beta || !idx || !counts) return MOE_ERR_INVALID_ARG;
  if ((m * int64_t(k)) % n != 0 || iters < 0 || !(gamma >= 0.f) || !isfinite(gamma)) return MOE_ERR_INVALID_ARG;
  if (n > 256 || k > kMaxK || m > 0x7FFFFFFFll || m * k > 0x7FFFFFFFll) return MOE_ERR_UNSUPPORTED;
  if (!ws_ok(ws, ws_bytes, moe_balance_workspace_size(m, n, k, 0))) return ws ? MOE_ERR_WORKSPACE : MOE_ERR_INVALID_ARG;
  BalanceArgs a{};
  a.m = m;
  a.n = n;
  a.k = k;
  a.q = m * k / n;
  a.s = s;
  a.beta = beta;
  a.iters = iters;
  a.idx = idx;
  a.counts = counts;
  a.ws = static_cast<char*>(ws) + kControlBytes;
  a.done = ctl_ticket(ws, kTicketBalance);
  a.nblocks = 1;
  a.beta_rows = m;
  return hip_status(launch_signsgd(a, gamma, static_cast<hipStream_t>(stream)));
}

moe_status moe_dispatch(const moe_shape* shape, int32_t capacity, const void* x, const int32_t* idx,
                        int32_t* token_to_row, uint8_t* drop_mask, int32_t* expert_offsets, int32_t* expert_rows,
                        int32_t* row_to_token, void* dispatched, void* ws, size_t ws_bytes, void* stream) {
  moe_status st = check_shape(shape);
  if (st != MOE_OK) return st;
  if (capacity < -1 || !idx || !token_to_row || !expert_offsets) return MOE_ERR_INVALID_ARG;
  if (dispatched && !x) return MOE_ERR_INVALID_ARG;
  const Layout L = layout(*shape, capacity, 0);
  if (!ws_ok(ws, ws_bytes, L.dispatch_end)) return ws ? MOE_ERR_WORKSPACE : MOE_ERR_INVALID_ARG;
  return do_dispatch(*shape, L, capacity, x, idx, token_to_row, drop_mask, expert_offsets, expert_rows, row_to_token,
                     dispatched, ws, false, static_cast<hipStream_t>(stream));
}

size_t moe_expert_ffn_workspace_size(int32_t n, int32_t rows_max, int32_t d_ff) {
  if (n < 1 || rows_max < 0 || d_ff < 1) return 0;
  return kControlBytes + al(ffn_ws_bytes(int64_t(n) * rows_max, d_ff));
}

moe_status moe_expert_weights_pack(int32_t n, int32_t rows, int32_t cols, const void* w, void* w_packed,
                                   void* stream) {
  if (n < 1 || rows < 1 || cols < 1 || !w || !w_packed || w == w_packed) return MOE_ERR_INVALID_ARG;
  if (rows % 32 != 0 || cols % 64 != 0 || n > kMaxExperts) return MOE_ERR_UNSUPPORTED;
  if ((reinterpret_cast<uintptr_t>(w) | reinterpret_cast<uintptr_t>(w_packed)) % 16 != 0) return MOE_ERR_INVALID_ARG;
  return hip_status(launch_pack_weights(n, rows, cols, static_cast<const uint16_t*>(w),
                                        static_cast<uint16_t*>(w_packed), static_cast<hipStream_t>(stream)));
}

moe_status moe_expert_ffn(int32_t n, int32_t d, int32_t d_ff, int32_t rows_max, const int32_t* expert_offsets,
                          const int32_t* expert_rows, const void* dispatched, const void* w1, const void* w2, void* y,
                          void* ws, size_t ws_bytes, void* stream) {
  if (n < 1 || d < 1 || d_ff < 1 || rows_max < 0 || !expert_offsets || !dispatched || !w1 || !w2 || !y)
    return MOE_ERR_INVALID_ARG;
  if (d % 32 != 0 || d_ff % 32 != 0 || n > kMaxExperts) return MOE_ERR_UNSUPPORTED;
  if (!ws_ok(ws, ws_bytes, moe_expert_ffn_workspace_size(n, rows_max, d_ff)))
    return ws ? MOE_ERR_WORKSPACE : MOE_ERR_INVALID_ARG;
  return hip_status(launch_expert_ffn(n, d, d_ff, rows_max, expert_offsets, expert_rows,
                                      static_cast<const uint16_t*>(dispatched),
                                      static_cast<const uint16_t*>(w1), static_cast<const uint16_t*>(w2),
                                      at<uint16_t>(ws, kControlBytes), static_cast<uint16_t*>(y),
                                      static_cast<hipStream_t>(stream)));
}

moe_status moe_combine(const moe_shape* shape, const void* y, int32_t y_dtype, const float* gate,
                       const int32_t* token_to_row, const void* residual, void* out, void* stream) {
  moe_status st = check_shape(shape);
  if (st != MOE_OK) return st;
  if (!y || !gate || !token_to_row || !out || (y_dtype != MOE_F32 && y_dtype != MOE_BF16)) return MOE_ERR_INVALID_ARG;
  return hip_status(launch_combine(shape->m, shape->d, shape->k, y, y_dtype == MOE_BF16, gate, token_to_row, residual,
                                   out, shape->x_dtype == MOE_BF16, static_cast<hipStream_t>(stream)));
}

moe_status moe_switch_layer(const moe_shape* shape, const moe_layer_params* p, const void* x, const float* w_r,
                            const void* w1, const void* w2, const float* bias, const moe_layer_outputs* o, void* ws,
                            size_t ws_bytes, void* stream) {
  moe_status st = check_shape(shape);
  if (st != MOE_OK) return st;
  if (!p || !o || !x || !w_r || !o->out || p->capacity < -1) return MOE_ERR_INVALID_ARG;
  const bool ffn = p->expert_kind == MOE_EXPERT_RELU_FFN;
  if (!ffn && p->expert_kind != MOE_EXPERT_IDENTITY) return MOE_ERR_INVALID_ARG;
  if (ffn && (!w1 || !w2 || p->d_ff < 1 || shape->x_dtype != MOE_BF16)) return MOE_ERR_INVALID_ARG;
  if (ffn && (shape->d % 32 != 0 || p->d_ff % 32 != 0)) return MOE_ERR_UNSUPPORTED;
  if (p->weights_packed && !ffn) return MOE_ERR_INVALID_ARG;
  // the bias the layer updates is the one it routes with, after the routing
  if (p->update_bias && (p->update_bias != bias || !isfinite(p->gamma))) return MOE_ERR_INVALID_ARG;
  if ((p->global_counts == nullptr) != (p->global_tokens == nullptr)) return MOE_ERR_INVALID_ARG;
  const Layout L = layout(*shape, p->capacity, ffn ? p->d_ff : 0);
  if (!ws_ok(ws, ws_bytes, L.total)) return ws ? MOE_ERR_WORKSPACE : MOE_ERR_INVALID_ARG;
  if (p->weights_packed &&
      (!ffn_packed_ok(shape->d, p->d_ff, effective_capacity(p->capacity, L.pairs), shape->n) ||
       (reinterpret_cast<uintptr_t>(w1) | reinterpret_cast<uintptr_t>(w2)) % 16 != 0))
    return MOE_ERR_UNSUPPORTED;
  hipStream_t s = static_cast<hipStream_t>(stream);
  const moe_shape& sh = *shape;
  int32_t* idx = o->idx ? o->idx : at<int32_t>(ws, L.idx);
  float* gate = o->gate ? o->gate : at<float>(ws, L.gate);
  int32_t* counts = o->counts ? o->counts : at<int32_t>(ws, L.counts);
  float* psum = o->prob_sum ? o->prob_sum : at<float>(ws, L.psum);
  float* f = o->f ? o->f : at<float>(ws, L.f);
  float* P = o->P ? o->P : at<float>(ws, L.P);
  float* aux = o->aux ? o->aux : at<float>(ws, L.aux);
  int32_t* t2r = o->token_to_row ? o->token_to_row : at<int32_t>(ws, L.t2r);
  uint8_t* drop = o->drop_mask ? o->drop_mask : at<uint8_t>(ws, L.drop);
  int32_t* offs = o->expert_offsets ? o->expert_offsets : at<int32_t>(ws, L.offs);
  int32_t* rowsn = o->expert_rows ? o->expert_rows : at<int32_t>(ws, L.rowsn);
  void* disp = o->dispatched ? o->dispatched : at<void>(ws, L.disp);
  void* y = ffn ? (o->y ? o->y : at<void>(ws, L.y)) : disp;

  auto mark = [&](int i) {
    if (p->stage_events && p->stage_events[i]) hipEventRecord(static_cast<hipEvent_t>(p->stage_events[i]), s);
  };
  // route (+ load statistics + per-chunk counts and capacity prefix sums in its last workgroup), then
  // slots + permute-dispatch in one kernel
  DispatchArgs da = dispatch_args(sh, L, p->capacity, x, idx, t2r, drop, offs, rowsn, o->row_to_token, disp, ws);
  RouteExtras ex;
  ex.f = f;
  ex.P = P;
  ex.aux = aux;
  ex.alpha = p->alpha;
  const bool fused_prefix = L.disp_ct == L.route_ct;
  if (fused_prefix && L.rp.fused && dispatch_self_prefix_ok(L.nch, sh.n)) {
    // the route kernel stops after its chunk rows; the dispatch workgroups derive
    // the totals, slot bases and offsets, and publish the load statistics
    ex.defer_finish = true;
    da.self_prefix = true;
    da.sup_counts = at<int32_t>(ws, kSupCountsOff);
    da.sup_psum = at<unsigned long long>(ws, kSupPsumOff);
    da.counts = counts;
    da.prob_sum = psum;
    da.f = f;
    da.P = P;
    da.aux = aux;
    da.alpha = p->alpha;
    da.gcounts = p->global_counts;
    da.gtokens = p->global_tokens;
    da.lf_bias = p->update_bias;
    da.gamma = p->gamma;
  } else {
    // the route's last workgroup publishes the statistics: it also takes the
    // global-batch accumulation and the bias update
    if (fused_prefix) ex.disp = &da;
    ex.gcounts = p->global_counts;
    ex.gtokens = p->global_tokens;
    ex.lf_bias = p->update_bias;
    ex.gamma = p->gamma;
  }
  mark(0);
  const void* planes = nullptr;   // else the route kernel splits W_r itself
  if (L.rp.mfma && !route_direct(L.rp, sh.d, sh.n) && (reinterpret_cast<uintptr_t>(x) % 16) == 0) {
    if ((st = hip_status(launch_router_prepare(L.rp, sh.d, sh.n, w_r, at<uint16_t>(ws, L.planes), s))) != MOE_OK)
      return st;
    planes = at<void>(ws, L.planes);
  }
  mark(1);
  // After the route kernel has added into the per-super-chunk control words, only the
  // combine clears them: a launch that fails before it clears them here, so that the
  // workspace stays usable for the next call.
  auto fail = [&](moe_status e) {
    if (da.self_prefix) zero_bytes(at<char>(ws, kSupCountsOff), kControlBytes - kSupCountsOff, s);
    return e;
  };
  if ((st = do_route(sh, L, x, w_r, planes, bias, idx, gate, counts, psum, ws, s, ex)) != MOE_OK) return fail(st);
  mark(2);
  if ((st = hip_status(launch_dispatch(da, fused_prefix, s))) != MOE_OK) return fail(st);
  mark(3);
  if (ffn) {
    const int32_t rows_max = effective_capacity(p->capacity, L.pairs);
    if ((st = hip_status(launch_expert_ffn(sh.n, sh.d, p->d_ff, rows_max, offs, da.padded ? rowsn : nullptr,
                                           static_cast<const uint16_t*>(disp),
                                           static_cast<const uint16_t*>(w1), static_cast<const uint16_t*>(w2),
                                           o->hidden ? static_cast<uint16_t*>(o->hidden) : at<uint16_t>(ws, L.hidden),
                                           static_cast<uint16_t*>(y), s, p->weights_packed != 0))) != MOE_OK)
      return fail(st);
  }
  mark(4);
  // the combine also clears the per-super-chunk sums for the next layer call
  st = hip_status(launch_combine(sh.m, sh.d, sh.k, y, ffn ? true : sh.x_dtype == MOE_BF16, gate, t2r, x, o->out,
                                 sh.x_dtype == MOE_BF16, s, da.self_prefix ? at<void>(ws, kSupCountsOff) : nullptr,
                                 kControlBytes - kSupCountsOff));
  if (st != MOE_OK) return fail(st);
  mark(5);
  return st;
}

size_t moe_switch_layer_backward_workspace_size(const moe_shape* shape, int32_t capacity, int32_t d_ff) {
  if (check_shape(shape) != MOE_OK || capacity < -1 || d_ff < 1) return 0;
  const int64_t pairs = shape->m * shape->k;
  const int64_t rows_bound = capacity < 0 ? pairs : int64_t(capacity) * shape->n;
  return kControlBytes + al(backward_ws_bytes(shape->m, shape->d, shape->n, shape->k, rows_bound, d_ff));
}

moe_status moe_switch_layer_backward(const moe_shape* shape, const moe_layer_params* p, const void* x,
                                     const float* w_r, const void* w1, const void* w2, const moe_layer_saved* sv,
                                     const float* dout, const moe_layer_grads* gr, void* ws, size_t ws_bytes,
                                     void* stream) {
  moe_status st = check_shape(shape);
  if (st != MOE_OK) return st;
  if (!p || !x || !w_r || !w1 || !w2 || !sv || !dout || !gr || p->capacity < -1 || p->d_ff < 1)
    return MOE_ERR_INVALID_ARG;
  if (!sv->idx || !sv->gate || !sv->counts || !sv->token_to_row || !sv->expert_offsets || !sv->dispatched ||
      !sv->hidden || !sv->y || !gr->dx || !gr->dw_r || !gr->dw1 || !gr->dw2)
    return MOE_ERR_INVALID_ARG;
  if (p->expert_kind != MOE_EXPERT_RELU_FFN || shape->x_dtype != MOE_BF16 || p->weights_packed)
    return MOE_ERR_INVALID_ARG;
  if (shape->score != MOE_SCORE_SOFTMAX || shape->gate != MOE_GATE_PROB) return MOE_ERR_UNSUPPORTED;
  if (shape->d % 32 != 0 || p->d_ff % 32 != 0) return MOE_ERR_UNSUPPORTED;
  if (!ws_ok(ws, ws_bytes, moe_switch_layer_backward_workspace_size(shape, p->capacity, p->d_ff)))
    return ws ? MOE_ERR_WORKSPACE : MOE_ERR_INVALID_ARG;
  const int64_t pairs = shape->m * shape->k;
  BackwardArgs b{};
  b.m = shape->m;
  b.d = shape->d;
  b.n = shape->n;
  b.k = shape->k;
  b.d_ff = p->d_ff;
  b.rows_bound = p->capacity < 0 ? pairs : int64_t(p->capacity) * shape->n;
  b.rows_max = effective_capacity(p->capacity, pairs);
  b.x_bf16 = true;
  b.alpha = p->alpha;
  b.x = x;
  b.w_r = w_r;
  b.w1 = static_cast<const uint16_t*>(w1);
  b.w2 = static_cast<const uint16_t*>(w2);
  b.idx = sv->idx;
  b.gate = sv->gate;
  b.counts = sv->counts;
  b.t2r = sv->token_to_row;
  b.offsets = sv->expert_offsets;
  b.rows = sv->expert_rows;
  b.dispatched = static_cast<const uint16_t*>(sv->dispatched);
  b.hidden = static_cast<const uint16_t*>(sv->hidden);
  b.y = static_cast<const uint16_t*>(sv->y);
  b.dout = dout;
  b.dx = gr->dx;
  b.dw_r = gr->dw_r;
  b.dw1 = gr->dw1;
  b.dw2 = gr->dw2;
  b.ws = static_cast<char*>(ws) + kControlBytes;
  return hip_status(launch_backward(b, static_cast<hipStream_t>(stream)));
}

}  // extern "C"
