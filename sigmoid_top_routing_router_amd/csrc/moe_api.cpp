// C ABI of the MoE layer library: argument checks, workspace carving and the
// launch sequence on the caller's stream.  No allocation, no host/device
// synchronisation, no device-to-host copies.
#include <cmath>
#include <cstddef>
#include <hip/hip_runtime.h>

#include <cstdarg>
#include <cstdio>
#include <mutex>
#include <string>
#include <vector>

#include "../../include/moe_mi355x.h"
#include "api_internal.h"
#include "kernels.h"

namespace {

thread_local std::string g_err;

moe_status_t fail(moe_status_t s, const char* fmt, ...) {
  char buf[512];
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(buf, sizeof(buf), fmt, ap);
  va_end(ap);
  g_err = buf;
  return s;
}

moe_status_t ok() {
  g_err.clear();
  return MOE_OK;
}

moe_status_t hip_fail(hipError_t e, const char* where) {
  return fail(MOE_ERR_HIP, "%s: %s", where, hipGetErrorString(e));
}

bool aligned(const void* p, size_t a) { return ((uintptr_t)p % a) == 0; }

constexpr int64_t kMaxN = int64_t(1) << 24;
constexpr size_t kAlign = 256;

size_t up(size_t v) { return (v + kAlign - 1) / kAlign * kAlign; }

// Sequential carve of one workspace; sizes rounded up to 256 bytes.
struct Carver {
  char* base;
  size_t off = 0;
  explicit Carver(void* b) : base((char*)b) {}
  template <class T>
  T* take(size_t count) {
    T* p = base ? (T*)(base + off) : nullptr;
    off += up(count * sizeof(T));
    return p;
  }
};

moe_status_t check_route_shape(int64_t N, int32_t E, int32_t K) {
  if (N < 1 || N > kMaxN) return fail(MOE_ERR_UNSUPPORTED_SHAPE, "N=%lld outside [1, 2^24]", (long long)N);
  if (K < 1 || K > MOE_MAX_K) return fail(MOE_ERR_UNSUPPORTED_SHAPE, "K=%d outside [1, %d]", K, MOE_MAX_K);
  if (E <= K || E > MOE_MAX_E) return fail(MOE_ERR_UNSUPPORTED_SHAPE, "E=%d must satisfy K < E <= %d", E, MOE_MAX_E);
  return MOE_OK;
}

// Workspace of the EQB update (histograms, selection state, raw quantiles,
// and the token bias when it has to be computed).
struct EqbLayout {
  uint32_t* hist;
  uint32_t* state;
  float* qraw;
  float* alpha;
};
EqbLayout carve_eqb(Carver& c, int64_t N, int E, int key_bits) {
  EqbLayout l;
  l.hist = c.take<uint32_t>(moe::eqb_hist_bytes(E, key_bits) / 4);
  l.state = c.take<uint32_t>(moe::eqb_state_bytes(E) / 4);
  l.qraw = c.take<float>((size_t)E);
  l.alpha = c.take<float>((size_t)N);
  return l;
}

struct FwdLayout {
  float* Z;
  int32_t* ids0;
  float* alpha;
  int32_t* ids;
  float* S;
  float* margin;
  float* beta_new;
  int32_t* counts_before;
  EqbLayout eqb;
  uint32_t* block_counts;
  int32_t* counts;
  int32_t* offsets;
  int32_t* sorted_src;
  int32_t* src_pos;
  int32_t* tiles;
  int32_t* n_tiles;
  uint16_t* H;
  uint16_t* Hs;
  uint16_t* Y;
  uint16_t* sh;
  // FP8 experts: x, H and the shared H as E4M3 codes with 1 x 128 scales
  uint8_t* xq;
  float* xs;
  uint8_t* Hq;
  float* Hqs;
  uint8_t* Hsq;
  float* Hss;
  float* part;       // split-K partial sums of the dense products of a small batch
  float* part_side;  // the same for the shared expert on the side stream
  size_t bytes;
  int64_t max_tiles;
};

// A batch of at most 64 tokens whose shared expert has the routed experts'
// hidden width runs that expert as up to four more m-tiles (16 rows each)
// of the weight-streaming products (no side stream, no launches of its own).
static bool shared_folded(const moe_problem_t& p) {
  return p.N <= moe::kSmallBatch && p.n_shared == 1 && p.h_shared == p.h;
}

FwdLayout carve_forward(void* ws, const moe_problem_t& p, bool fp8 = false) {
  Carver c(ws);
  FwdLayout l{};
  const int64_t N = p.N, pairs = p.N * (int64_t)p.K;
  const int key_bits = (p.flags & MOE_KEY32) ? 32 : 16;
  // the shared expert folded into the weight-streaming products: N more
  // rows of H and Y, at most four more m-tiles of 16 rows
  const int64_t hy_rows = pairs + (shared_folded(p) ? N : 0);
  l.Z = c.take<float>((size_t)N * p.E);
  l.ids0 = c.take<int32_t>((size_t)pairs);
  l.alpha = c.take<float>((size_t)N);
  l.ids = c.take<int32_t>((size_t)pairs);
  l.S = c.take<float>((size_t)pairs);
  l.margin = c.take<float>((size_t)N);
  l.beta_new = c.take<float>((size_t)p.E);
  l.counts_before = c.take<int32_t>((size_t)p.E);
  l.eqb = carve_eqb(c, N, p.E, key_bits);
  l.block_counts = c.take<uint32_t>((size_t)moe::perm_count_rows(pairs) * p.E);
  l.counts = c.take<int32_t>((size_t)p.E);
  l.offsets = c.take<int32_t>((size_t)p.E + 1);
  l.sorted_src = c.take<int32_t>((size_t)pairs);
  l.src_pos = c.take<int32_t>((size_t)pairs);
  l.max_tiles = moe::perm_max_tiles(pairs, p.E, moe::gemm_bm()) + (shared_folded(p) ? 4 : 0);
  l.tiles = c.take<int32_t>((size_t)l.max_tiles * 4);
  l.n_tiles = c.take<int32_t>(4);
  if (fp8) {
    l.xq = c.take<uint8_t>((size_t)N * p.d);
    l.xs = c.take<float>((size_t)N * (p.d / 128));
    l.Hq = c.take<uint8_t>((size_t)hy_rows * p.h);
    l.Hqs = c.take<float>((size_t)hy_rows * (p.h / 128));
  } else {
    l.H = c.take<uint16_t>((size_t)hy_rows * p.h);
  }
  l.Y = c.take<uint16_t>((size_t)hy_rows * p.d);
  if (p.n_shared > 0) {
    if (fp8) {
      l.Hsq = c.take<uint8_t>((size_t)N * p.h_shared);
      l.Hss = c.take<float>((size_t)N * (p.h_shared / 128));
    } else {
      l.Hs = c.take<uint16_t>((size_t)N * p.h_shared);
    }
    l.sh = c.take<uint16_t>((size_t)N * p.d);
  }
  if (N <= moe::kSmallBatch) {
    l.part = c.take<float>(moe::dense_small_part_floats(N, p.d, p.E, p.n_shared ? p.h_shared : 0));
    if (p.n_shared > 0)
      l.part_side = c.take<float>(moe::dense_small_part_floats(N, p.d, 0, p.h_shared));
  }
  l.bytes = c.off;
  return l;
}

moe_status_t check_problem(const moe_problem_t* p) {
  if (!p) return fail(MOE_ERR_INVALID_ARGUMENT, "problem is NULL");
  moe_status_t s = check_route_shape(p->N, p->E, p->K);
  if (s != MOE_OK) return s;
  if (p->d < 64 || p->d > 8192 || p->d % 64)
    return fail(MOE_ERR_UNSUPPORTED_SHAPE, "d=%d must be a multiple of 64 in [64, 8192]", p->d);
  if (p->h < 32 || p->h > 4096 || p->h % 32)
    return fail(MOE_ERR_UNSUPPORTED_SHAPE, "h=%d must be a multiple of 32 in [32, 4096]", p->h);
  if (p->n_shared != 0 && p->n_shared != 1)
    return fail(MOE_ERR_UNSUPPORTED_SHAPE, "n_shared=%d must be 0 or 1", p->n_shared);
  if (p->n_shared == 1 && (p->h_shared < 32 || p->h_shared > 4096 || p->h_shared % 32))
    return fail(MOE_ERR_UNSUPPORTED_SHAPE, "h_shared=%d must be a multiple of 32 in [32, 4096]", p->h_shared);
  // the GEMMs address x, H and the shared H with 32-bit byte offsets
  const uint64_t lim = 0xFFFFFFFFull;
  if ((uint64_t)p->N * (uint64_t)p->d * 2u > lim ||
      (uint64_t)p->N * (uint64_t)p->K * (uint64_t)p->h * 2u > lim ||
      (p->n_shared == 1 && (uint64_t)p->N * (uint64_t)p->h_shared * 2u > lim))
    return fail(MOE_ERR_UNSUPPORTED_SHAPE,
                "N=%lld too large: x [N,d], the routed hidden rows [N*K,h] and the shared "
                "hidden rows [N,h_shared] must each be below 4 GiB in bf16",
                (long long)p->N);
  if (p->flags & ~(MOE_RECOMPUTE_BIAS | MOE_KEY32 | MOE_PACKED_GATEUP | MOE_ROUTE_FUSED))
    return fail(MOE_ERR_INVALID_ARGUMENT, "unknown flag bits 0x%x", p->flags);
  if (p->logits_in && p->logit_offset)
    return fail(MOE_ERR_INVALID_ARGUMENT, "logit_offset applies to computed logits only; logits_in is set");
  if (p->logits_in && !aligned(p->logits_in, 4)) return fail(MOE_ERR_INVALID_ARGUMENT, "logits_in misaligned");
  if (p->logit_offset && !aligned(p->logit_offset, 4)) return fail(MOE_ERR_INVALID_ARGUMENT, "logit_offset misaligned");
  return MOE_OK;
}

// The FP8 path quantises in 1 x 128 groups and multiplies 128 x 128 blocks.
moe_status_t check_problem_fp8(const moe_problem_t* p) {
  moe_status_t s = check_problem(p);
  if (s != MOE_OK) return s;
  if (p->d % 128 || p->h % 128 || (p->n_shared == 1 && p->h_shared % 128))
    return fail(MOE_ERR_UNSUPPORTED_SHAPE,
                "FP8 experts need d, h and h_shared to be multiples of 128 (d=%d h=%d hs=%d)",
                p->d, p->h, p->h_shared);
  return MOE_OK;
}

// Expert weights of one forward call: bf16 (moe_weights_t) or E4M3 codes
// with block scales (moe_fp8_weights_t).
struct Experts {
  bool fp8 = false;
  // everything on the caller's stream, no stage timing: no stream or event
  // is ever created by the call
  bool in_order = false;
  const uint16_t* w_router = nullptr;
  const moe_weights_t* b = nullptr;
  const moe_fp8_weights_t* q = nullptr;
};

// ---- stage timing: S+1 boundary events per recorded call
constexpr int kGateUpStage = 3;  // the routed gate/up GEMM
struct StageTimer {
  std::mutex mu;
  bool enabled = false;
  bool gateup_only = false;      // record only the boundaries of stage 3
  std::vector<hipEvent_t> pool;  // reused across reads
  size_t used = 0;               // events recorded since the last read
};
StageTimer g_timer;

struct CallTimer {
  bool on = false;
  bool gateup_only = false;
  size_t base = 0;
  int next = 0;
  hipStream_t st = nullptr;
  hipError_t start(hipStream_t s) {
    {
      std::lock_guard<std::mutex> g(g_timer.mu);
      if (!g_timer.enabled) return hipSuccess;
      on = true;
      gateup_only = g_timer.gateup_only;
      st = s;
      base = g_timer.used;
      g_timer.used += MOE_NUM_STAGES + 1;
      while (g_timer.pool.size() < g_timer.used) {
        hipEvent_t e;
        hipError_t err = hipEventCreate(&e);
        if (err != hipSuccess) return err;
        g_timer.pool.push_back(e);
      }
    }
    return mark();  // takes the lock itself
  }
  // Record the boundary after the current stage.
  hipError_t mark() {
    if (!on) return hipSuccess;
    const int b = next++;
    if (gateup_only && b != kGateUpStage && b != kGateUpStage + 1) return hipSuccess;
    hipEvent_t e;
    {
      std::lock_guard<std::mutex> g(g_timer.mu);
      e = g_timer.pool[base + b];
    }
    return hipEventRecord(e, st);
  }
};

// The shared expert does not depend on the routing, so at batch sizes that
// use the tile engine its two products run on a second stream, next to the
// router GEMM, the routing, the grouping and the routed experts, filling the
// compute units those leave idle.  One non-blocking stream (default
// priority) and its fork and join events per device and host thread, created
// on first use and kept until the process ends; where they cannot be created
// the products run in order on the caller's stream instead.
struct SideStream {
  hipStream_t s = nullptr;
  hipEvent_t fork = nullptr, join = nullptr;
  bool failed = false;
};
constexpr int kMaxSideDevices = 64;

SideStream* side_stream() {
  thread_local SideStream tab[kMaxSideDevices];
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxSideDevices) {
    (void)hipGetLastError();
    return nullptr;
  }
  SideStream& t = tab[dev];
  if (t.failed) return nullptr;
  if (!t.s) {
    if (hipStreamCreateWithFlags(&t.s, hipStreamNonBlocking) != hipSuccess ||
        hipEventCreateWithFlags(&t.fork, hipEventDisableTiming) != hipSuccess ||
        hipEventCreateWithFlags(&t.join, hipEventDisableTiming) != hipSuccess) {
      (void)hipGetLastError();
      t.failed = true;
      return nullptr;
    }
  }
  return &t;
}

// Makes the caller's stream wait for the side stream's work once, at the
// latest when it goes out of scope (also on an error return, so that a
// captured graph never holds an unjoined branch).
struct SideJoin {
  hipStream_t st = nullptr;
  SideStream* side = nullptr;
  hipError_t join() {
    if (!side) return hipSuccess;
    SideStream* t = side;
    side = nullptr;
    return hipStreamWaitEvent(st, t->join, 0);
  }
  ~SideJoin() { (void)join(); }
};

#define MOE_TRY_HIP(expr, where)                   \
  do {                                             \
    hipError_t _e = (expr);                        \
    if (_e != hipSuccess) return hip_fail(_e, where); \
  } while (0)

}  // namespace

// The layer for either expert precision.  Shape and weight checks are the
// callers'; everything else is common.
static moe_status_t forward_impl(const moe_problem_t* p, const Experts& ex, const uint16_t* x,
                                 const float* beta_in, uint16_t* y, moe_aux_t* aux,
                                 void* workspace, size_t workspace_bytes, void* stream) {
  if (!p->logits_in && !ex.w_router)
    return fail(MOE_ERR_INVALID_ARGUMENT, "w_router is required when logits_in is NULL");
  if (!aligned(x, 16) || !aligned(y, 16))
    return fail(MOE_ERR_INVALID_ARGUMENT, "x and y must be 16-byte aligned");
  if (beta_in && !aligned(beta_in, 4)) return fail(MOE_ERR_INVALID_ARGUMENT, "beta_in misaligned");
  moe_aux_t none{};
  const moe_aux_t& A = aux ? *aux : none;
  const void* pa[] = {A.logits, A.topk_ids, A.topk_weights, A.alpha, A.margin, A.beta_out,
                      A.quantile_out, A.counts_before, A.counts, A.offsets, A.sorted_src,
                      A.src_pos};
  for (const void* q : pa)
    if (q && !aligned(q, 4)) return fail(MOE_ERR_INVALID_ARGUMENT, "aux buffers must be 4-byte aligned");
  const FwdLayout need = carve_forward(nullptr, *p, ex.fp8);
  if (!workspace || !aligned(workspace, kAlign))
    return fail(MOE_ERR_INVALID_ARGUMENT, "workspace must be non-NULL and 256-byte aligned");
  if (workspace_bytes < need.bytes)
    return fail(MOE_ERR_WORKSPACE_TOO_SMALL, "workspace %zu < required %zu", workspace_bytes, need.bytes);

  FwdLayout l = carve_forward(workspace, *p, ex.fp8);
  const moe_weights_t* w = ex.b;
  const moe_fp8_weights_t* q = ex.q;
  const hipStream_t st = (hipStream_t)stream;
  const int64_t N = p->N;
  const int E = p->E, K = p->K, d = p->d, h = p->h;
  const int key_bits = (p->flags & MOE_KEY32) ? 32 : 16;
  const bool recompute = (p->flags & MOE_RECOMPUTE_BIAS) != 0;

  CallTimer tm;
  if (!ex.in_order) MOE_TRY_HIP(tm.start(st), "moe_forward: stage timer");

  // Router logits and the shared expert's gate/up: on one stream both read
  // x, so they share one launch; with the side stream the shared expert runs
  // there instead.  FP8 experts first quantise x per 1 x 128 group; the
  // router reads the bf16 x.
  const float* Z;
  const bool shared = p->n_shared == 1;
  const int hs = p->h_shared;
  // A batch of at most 64 tokens reads every touched weight once and does
  // little arithmetic: its routed GEMMs stream the weights straight into
  // registers, and its dense products are split over many small blocks.
  const bool small = N <= moe::kSmallBatch;
  if (ex.fp8)
    MOE_TRY_HIP(moe::launch_quant_rows(x, N, d, l.xq, l.xs, st), "moe_forward: quantise x");
  SideJoin sj;
  const bool folded = shared_folded(*p);
  SideStream* side = (shared && !folded && !ex.in_order) ? side_stream() : nullptr;
  // the side stream starts from the caller's stream as it stands before the
  // router GEMM (the fork), but its work is enqueued after that GEMM, whose
  // blocks are then dispatched first
  if (side) MOE_TRY_HIP(hipEventRecord(side->fork, st), "moe_forward: fork");
  // Selection inside the router GEMM's epilogue (MOE_ROUTE_FUSED): the
  // tiles' candidate lists ([N][tiles][K+1] scores, then experts) live in the
  // expert-output buffer Y, which nothing reads or writes before the down
  // projection.
  moe::RouterSel rsel{};
  const moe::RouterSel* sel = nullptr;
  const int sel_tiles = moe::router_col_tiles(E);
  if (!small && !p->logits_in && (p->flags & MOE_ROUTE_FUSED)) {
    const size_t n = (size_t)N * sel_tiles * (K + 1);
    if (2 * n * sizeof(float) > (size_t)N * K * d * sizeof(uint16_t))
      return fail(MOE_ERR_UNSUPPORTED_SHAPE, "router selection lists do not fit");
    rsel = moe::RouterSel{beta_in, reinterpret_cast<float*>(l.Y),
                          reinterpret_cast<uint32_t*>(l.Y) + n, K};
    sel = &rsel;
  }
  // the shared expert's products on the caller's stream (no side stream)
  const bool shared_here = shared && !folded && !side;
  if (small) {
    if (p->logits_in) {
      Z = p->logits_in;
      if (A.logits)
        MOE_TRY_HIP(hipMemcpyAsync(A.logits, Z, (size_t)N * E * 4, hipMemcpyDeviceToDevice, st),
                    "moe_forward: logits copy");
    } else {
      float* zout = A.logits ? A.logits : l.Z;
      MOE_TRY_HIP(moe::launch_router_dense_small(x, ex.w_router, p->logit_offset, N, d, E, zout,
                                                 l.part, st),
                  "moe_forward: router GEMM");
      Z = zout;
    }
    if (shared_here && ex.fp8)
      MOE_TRY_HIP(moe::launch_shared_gateup_dense_small(l.xq, l.xs, N, d, q->ws_gate, q->ss_gate,
                                                        q->ws_up, q->ss_up, hs, true, l.Hsq,
                                                        l.Hss, l.part, st),
                  "moe_forward: shared gate/up");
    else if (shared_here)
      MOE_TRY_HIP(moe::launch_shared_gateup_dense_small(x, nullptr, N, d, w->ws_gate, nullptr,
                                                        w->ws_up, nullptr, hs, false, l.Hs,
                                                        nullptr, l.part, st),
                  "moe_forward: shared gate/up");
  } else if (p->logits_in) {
    Z = p->logits_in;
    if (A.logits)
      MOE_TRY_HIP(hipMemcpyAsync(A.logits, Z, (size_t)N * E * 4, hipMemcpyDeviceToDevice, st),
                  "moe_forward: logits copy");
    if (shared_here && ex.fp8)
      MOE_TRY_HIP(moe::launch_gateup_fp8(l.xq, l.xs, N, nullptr, 1, nullptr, nullptr, 0, N,
                                         q->ws_gate, q->ss_gate, q->ws_up, q->ss_up, d, hs,
                                         l.Hsq, l.Hss, st),
                  "moe_forward: shared gate/up");
    else if (shared_here)
      MOE_TRY_HIP(moe::launch_gateup(x, N, nullptr, 1, nullptr, nullptr, 0, N, w->ws_gate,
                                     w->ws_up, d, hs, l.Hs, st),
                  "moe_forward: shared gate/up");
  } else {
    float* zout = A.logits ? A.logits : l.Z;
    if (shared_here && ex.fp8)
      MOE_TRY_HIP(moe::launch_router_shared_gateup_fp8(x, l.xq, l.xs, N, d, ex.w_router,
                                                       p->logit_offset, E, zout, q->ws_gate,
                                                       q->ss_gate, q->ws_up, q->ss_up, hs,
                                                       l.Hsq, l.Hss, st, sel),
                  "moe_forward: router GEMM + shared gate/up");
    else if (shared_here)
      MOE_TRY_HIP(moe::launch_router_shared_gateup(x, N, d, ex.w_router, p->logit_offset, E,
                                                   zout, w->ws_gate, w->ws_up, hs, l.Hs, st,
                                                   sel),
                  "moe_forward: router GEMM + shared gate/up");
    else
      MOE_TRY_HIP(moe::launch_router_gemm(x, ex.w_router, p->logit_offset, N, d, E, zout, st,
                                          sel),
                  "moe_forward: router GEMM");
    Z = zout;
  }
  if (side) {
    // the shared expert on the side stream: gate/up, then down into l.sh,
    // which the combine reads after the join
    const hipStream_t s2 = side->s;
    MOE_TRY_HIP(hipStreamWaitEvent(s2, side->fork, 0), "moe_forward: fork");
    sj.st = st;
    sj.side = side;
    if (small) {
      // the split-K kernels of a small batch, with partial sums of their own
      if (ex.fp8)
        MOE_TRY_HIP(moe::launch_shared_gateup_dense_small(l.xq, l.xs, N, d, q->ws_gate,
                                                          q->ss_gate, q->ws_up, q->ss_up, hs,
                                                          true, l.Hsq, l.Hss, l.part_side, s2),
                    "moe_forward: shared gate/up");
      else
        MOE_TRY_HIP(moe::launch_shared_gateup_dense_small(x, nullptr, N, d, w->ws_gate, nullptr,
                                                          w->ws_up, nullptr, hs, false, l.Hs,
                                                          nullptr, l.part_side, s2),
                    "moe_forward: shared gate/up");
      MOE_TRY_HIP(moe::launch_shared_down_dense_small(
                      ex.fp8 ? (const void*)l.Hsq : (const void*)l.Hs, ex.fp8 ? l.Hss : nullptr,
                      N, d, ex.fp8 ? (const void*)q->ws_down : (const void*)w->ws_down,
                      ex.fp8 ? q->ss_down : nullptr, hs, ex.fp8, l.sh, l.part_side, s2),
                  "moe_forward: shared down");
    } else if (ex.fp8) {
      MOE_TRY_HIP(moe::launch_gateup_fp8(l.xq, l.xs, N, nullptr, 1, nullptr, nullptr, 0, N,
                                         q->ws_gate, q->ss_gate, q->ws_up, q->ss_up, d, hs,
                                         l.Hsq, l.Hss, s2),
                  "moe_forward: shared gate/up");
      MOE_TRY_HIP(moe::launch_down_fp8(l.Hsq, l.Hss, N, nullptr, nullptr, 0, N, q->ws_down,
                                       q->ss_down, d, hs, l.sh, s2),
                  "moe_forward: shared down");
    } else {
      MOE_TRY_HIP(moe::launch_gateup(x, N, nullptr, 1, nullptr, nullptr, 0, N, w->ws_gate,
                                     w->ws_up, d, hs, l.Hs, s2),
                  "moe_forward: shared gate/up");
      MOE_TRY_HIP(moe::launch_down(l.Hs, N, nullptr, nullptr, 0, N, w->ws_down, d, hs, l.sh, s2),
                  "moe_forward: shared down");
    }
    MOE_TRY_HIP(hipEventRecord(side->join, s2), "moe_forward: join");
  }
  MOE_TRY_HIP(tm.mark(), "moe_forward: stage timer");

  // selection, token bias, optional exact quantile update, re-route
  int32_t* ids = A.topk_ids ? A.topk_ids : l.ids;
  float* S = A.topk_weights ? A.topk_weights : l.S;
  float* alpha = A.alpha ? A.alpha : l.alpha;
  float* margin = A.margin ? A.margin : l.margin;
  if (recompute) {
    // first pass: alpha only, unless the loads before the update are wanted;
    // it also clears the first histogram of the quantile update
    if (sel)
      MOE_TRY_HIP(moe::launch_route_merge(sel->cand_s, sel->cand_e, sel_tiles, Z, N, E, K,
                                          A.counts_before ? l.ids0 : nullptr, nullptr, alpha,
                                          nullptr, st, l.eqb.hist, (size_t)E * 256),
                  "moe_forward: first routing");
    else
      MOE_TRY_HIP(moe::launch_route(Z, beta_in, N, E, K, A.counts_before ? l.ids0 : nullptr,
                                    nullptr, alpha, nullptr, st, l.eqb.hist, (size_t)E * 256),
                  "moe_forward: first routing");
    if (A.counts_before)
      MOE_TRY_HIP(moe::launch_count(l.ids0, N * K, E, A.counts_before, st), "moe_forward: loads");
    float* beta_new = A.beta_out ? A.beta_out : l.beta_new;
    moe::EqbWork ew{l.eqb.hist, l.eqb.state, l.eqb.qraw};
    // the centring of the raw quantiles happens inside the final routing pass
    MOE_TRY_HIP(moe::launch_eqb(Z, alpha, N, E, K, key_bits, nullptr, A.quantile_out, ew, st,
                                true),
                "moe_forward: quantile update");
    MOE_TRY_HIP(moe::launch_route_centred(Z, nullptr, l.eqb.qraw, beta_new, N, E, K, ids, S,
                                          nullptr, margin, st),
                "moe_forward: routing");
  } else if (sel) {
    MOE_TRY_HIP(moe::launch_route_merge(sel->cand_s, sel->cand_e, sel_tiles, Z, N, E, K, ids, S,
                                        alpha, margin, st),
                "moe_forward: routing");
    if (A.counts_before)
      MOE_TRY_HIP(moe::launch_count(ids, N * K, E, A.counts_before, st), "moe_forward: loads");
  } else {
    MOE_TRY_HIP(moe::launch_route(Z, beta_in, N, E, K, ids, S, alpha, margin, st),
                "moe_forward: routing");
    if (A.counts_before)
      MOE_TRY_HIP(moe::launch_count(ids, N * K, E, A.counts_before, st), "moe_forward: loads");
  }

  MOE_TRY_HIP(tm.mark(), "moe_forward: stage timer");

  // stable grouping by expert and the m-tile table
  moe::PermWork pw;
  pw.block_counts = l.block_counts;
  pw.counts = A.counts ? A.counts : l.counts;
  pw.offsets = A.offsets ? A.offsets : l.offsets;
  pw.sorted_src = A.sorted_src ? A.sorted_src : l.sorted_src;
  pw.src_pos = A.src_pos ? A.src_pos : l.src_pos;
  pw.tiles = l.tiles;
  pw.n_tiles = l.n_tiles;
  MOE_TRY_HIP(moe::launch_permute(ids, N, E, K, moe::gemm_bm(), moe::gemm_xrows(), pw, st,
                                  folded ? (int)N : 0),
              "moe_forward: grouping");
  MOE_TRY_HIP(tm.mark(), "moe_forward: stage timer");

  // routed experts (the gather is fused into the gate/up A loads)
  const bool packed = (p->flags & MOE_PACKED_GATEUP) != 0;
  const int64_t hy_rows = N * K + (folded ? N : 0);
  moe::SharedFold fold{};
  if (folded) {
    fold.gate = ex.fp8 ? (const void*)q->ws_gate : (const void*)w->ws_gate;
    fold.up = ex.fp8 ? (const void*)q->ws_up : (const void*)w->ws_up;
    fold.down = ex.fp8 ? (const void*)q->ws_down : (const void*)w->ws_down;
    fold.s_gate = ex.fp8 ? q->ss_gate : nullptr;
    fold.s_up = ex.fp8 ? q->ss_up : nullptr;
    fold.s_down = ex.fp8 ? q->ss_down : nullptr;
    fold.row0 = N * K;
  }
  const moe::SharedFold* sf = folded ? &fold : nullptr;
  if (ex.fp8 && small)
    MOE_TRY_HIP(moe::launch_gateup_fp8_small(l.xq, l.xs, N, pw.sorted_src, K, pw.tiles,
                                             pw.n_tiles, l.max_tiles, 0, q->w_gate, q->s_gate,
                                             q->w_up, q->s_up, d, h, l.Hq, l.Hqs, st, packed, sf),
                "moe_forward: gate/up");
  else if (ex.fp8)
    MOE_TRY_HIP(moe::launch_gateup_fp8(l.xq, l.xs, N, pw.sorted_src, K, pw.tiles, pw.n_tiles,
                                       l.max_tiles, 0, q->w_gate, q->s_gate, q->w_up, q->s_up, d,
                                       h, l.Hq, l.Hqs, st, packed),
                "moe_forward: gate/up");
  else if (small)
    MOE_TRY_HIP(moe::launch_gateup_small(x, N, pw.sorted_src, K, pw.tiles, pw.n_tiles,
                                         l.max_tiles, 0, w->w_gate, w->w_up, d, h, l.H, st,
                                         packed, sf),
                "moe_forward: gate/up");
  else
    MOE_TRY_HIP(moe::launch_gateup(x, N, pw.sorted_src, K, pw.tiles, pw.n_tiles, l.max_tiles, 0,
                                   w->w_gate, w->w_up, d, h, l.H, st, packed),
                "moe_forward: gate/up");
  MOE_TRY_HIP(tm.mark(), "moe_forward: stage timer");
  if (ex.fp8 && small)
    MOE_TRY_HIP(moe::launch_down_fp8_small(l.Hq, l.Hqs, hy_rows, pw.tiles, pw.n_tiles,
                                           l.max_tiles, 0, q->w_down, q->s_down, d, h, l.Y, st,
                                           sf),
                "moe_forward: down");
  else if (ex.fp8)
    MOE_TRY_HIP(moe::launch_down_fp8(l.Hq, l.Hqs, N * K, pw.tiles, pw.n_tiles, l.max_tiles, 0,
                                     q->w_down, q->s_down, d, h, l.Y, st),
                "moe_forward: down");
  else if (small)
    MOE_TRY_HIP(moe::launch_down_small(l.H, hy_rows, pw.tiles, pw.n_tiles, l.max_tiles, 0,
                                       w->w_down, d, h, l.Y, st, sf),
                "moe_forward: down");
  else
    MOE_TRY_HIP(moe::launch_down(l.H, N * K, pw.tiles, pw.n_tiles, l.max_tiles, 0, w->w_down, d,
                                 h, l.Y, st),
                "moe_forward: down");
  MOE_TRY_HIP(tm.mark(), "moe_forward: stage timer");
  // the shared expert's down projection
  if (shared_here && small)
    MOE_TRY_HIP(moe::launch_shared_down_dense_small(
                    ex.fp8 ? (const void*)l.Hsq : (const void*)l.Hs, ex.fp8 ? l.Hss : nullptr, N,
                    d, ex.fp8 ? (const void*)q->ws_down : (const void*)w->ws_down,
                    ex.fp8 ? q->ss_down : nullptr, hs, ex.fp8, l.sh, l.part, st),
                "moe_forward: shared down");
  else if (shared_here && ex.fp8)
    MOE_TRY_HIP(moe::launch_down_fp8(l.Hsq, l.Hss, N, nullptr, nullptr, 0, N, q->ws_down,
                                     q->ss_down, d, hs, l.sh, st), "moe_forward: shared down");
  else if (shared_here)
    MOE_TRY_HIP(moe::launch_down(l.Hs, N, nullptr, nullptr, 0, N, w->ws_down, d, hs, l.sh, st),
                "moe_forward: shared down");
  MOE_TRY_HIP(sj.join(), "moe_forward: join");
  MOE_TRY_HIP(tm.mark(), "moe_forward: stage timer");
  // weighted combine
  // the folded shared expert's output: rows N*K .. of Y, in token order
  const uint16_t* sh_out = folded ? l.Y + (size_t)N * K * d : (shared ? l.sh : nullptr);
  MOE_TRY_HIP(moe::launch_combine(sh_out, l.Y, S, pw.src_pos, N, K, d, y, st),
              "moe_forward: combine");
  MOE_TRY_HIP(tm.mark(), "moe_forward: stage timer");
  return ok();
}


extern "C" {

int32_t moe_abi_version(void) { return 2; }

moe_status_t moe_stage_timing(int32_t enable) {
  if (enable < 0 || enable > 2) return fail(MOE_ERR_INVALID_ARGUMENT, "enable=%d outside [0, 2]", enable);
  std::lock_guard<std::mutex> g(g_timer.mu);
  g_timer.enabled = enable != 0;
  g_timer.gateup_only = enable == 2;
  g_timer.used = 0;
  return ok();
}

moe_status_t moe_stage_times(double* ms, int64_t* calls) {
  if (!ms || !calls) return fail(MOE_ERR_INVALID_ARGUMENT, "ms and calls are required");
  std::lock_guard<std::mutex> g(g_timer.mu);
  for (int s = 0; s < MOE_NUM_STAGES; ++s) ms[s] = 0.0;
  const size_t per = MOE_NUM_STAGES + 1;
  const size_t n = g_timer.used / per;
  for (size_t c = 0; c < n; ++c) {
    hipEvent_t* ev = g_timer.pool.data() + c * per;
    if (g_timer.gateup_only) {
      MOE_TRY_HIP(hipEventSynchronize(ev[kGateUpStage + 1]), "moe_stage_times");
      float t = 0.0f;
      MOE_TRY_HIP(hipEventElapsedTime(&t, ev[kGateUpStage], ev[kGateUpStage + 1]),
                  "moe_stage_times");
      ms[kGateUpStage] += t;
      continue;
    }
    MOE_TRY_HIP(hipEventSynchronize(ev[MOE_NUM_STAGES]), "moe_stage_times");
    for (int s = 0; s < MOE_NUM_STAGES; ++s) {
      float t = 0.0f;
      MOE_TRY_HIP(hipEventElapsedTime(&t, ev[s], ev[s + 1]), "moe_stage_times");
      ms[s] += t;
    }
  }
  *calls = (int64_t)n;
  g_timer.used = 0;
  return ok();
}

const char* moe_stage_name(int32_t stage) {
  static const char* names[MOE_NUM_STAGES] = {"router_shared_gate_up", "routing", "grouping",
                                              "gate_up", "down", "shared_down", "combine"};
  return (stage >= 0 && stage < MOE_NUM_STAGES) ? names[stage] : "";
}

const char* moe_status_string(moe_status_t s) {
  switch (s) {
    case MOE_OK: return "MOE_OK";
    case MOE_ERR_INVALID_ARGUMENT: return "MOE_ERR_INVALID_ARGUMENT";
    case MOE_ERR_UNSUPPORTED_SHAPE: return "MOE_ERR_UNSUPPORTED_SHAPE";
    case MOE_ERR_WORKSPACE_TOO_SMALL: return "MOE_ERR_WORKSPACE_TOO_SMALL";
    case MOE_ERR_HIP: return "MOE_ERR_HIP";
  }
  return "MOE_ERR_UNKNOWN";
}

const char* moe_last_error_message(void) { return g_err.c_str(); }

moe_status_t moe_route(const float* logits, const float* beta, int64_t N, int32_t E,
                       int32_t K, int32_t* topk_ids, float* topk_weights, float* alpha,
                       float* margin, void* stream) {
  moe_status_t s = check_route_shape(N, E, K);
  if (s != MOE_OK) return s;
  if (!logits || !topk_ids || !topk_weights)
    return fail(MOE_ERR_INVALID_ARGUMENT, "logits, topk_ids and topk_weights are required");
  const void* ptrs[] = {logits, beta, topk_ids, topk_weights, alpha, margin};
  for (const void* q : ptrs)
    if (q && !aligned(q, 4)) return fail(MOE_ERR_INVALID_ARGUMENT, "pointer not 4-byte aligned");
  MOE_TRY_HIP(moe::launch_route(logits, beta, N, E, K, topk_ids, topk_weights, alpha, margin,
                                (hipStream_t)stream), "moe_route");
  return ok();
}

size_t moe_eqb_workspace_bytes(int64_t N, int32_t E, int32_t key_bits) {
  if (N < 1 || E < 1 || (key_bits != 16 && key_bits != 32)) return 0;
  Carver c(nullptr);
  carve_eqb(c, N, E, key_bits);
  return c.off;
}

moe_status_t moe_eqb_bias(const float* logits, const float* beta_in, const float* alpha,
                          int64_t N, int32_t E, int32_t K, int32_t key_bits, float* beta_out,
                          float* quantile_out, void* workspace, size_t workspace_bytes,
                          void* stream) {
  moe_status_t s = check_route_shape(N, E, K);
  if (s != MOE_OK) return s;
  if (key_bits != 16 && key_bits != 32)
    return fail(MOE_ERR_INVALID_ARGUMENT, "key_bits=%d must be 16 or 32", key_bits);
  if (!logits || !beta_out) return fail(MOE_ERR_INVALID_ARGUMENT, "logits and beta_out are required");
  const void* ptrs[] = {logits, beta_in, alpha, beta_out, quantile_out};
  for (const void* q : ptrs)
    if (q && !aligned(q, 4)) return fail(MOE_ERR_INVALID_ARGUMENT, "pointer not 4-byte aligned");
  const size_t need = moe_eqb_workspace_bytes(N, E, key_bits);
  if (!workspace || !aligned(workspace, kAlign))
    return fail(MOE_ERR_INVALID_ARGUMENT, "workspace must be non-NULL and 256-byte aligned");
  if (workspace_bytes < need)
    return fail(MOE_ERR_WORKSPACE_TOO_SMALL, "workspace %zu < required %zu", workspace_bytes, need);
  Carver c(workspace);
  EqbLayout l = carve_eqb(c, N, E, key_bits);
  const hipStream_t st = (hipStream_t)stream;
  const float* a = alpha;
  if (!a) {
    // the routing that gives alpha also clears the first histogram
    MOE_TRY_HIP(moe::launch_route(logits, beta_in, N, E, K, nullptr, nullptr, l.alpha, nullptr, st,
                                  l.hist, (size_t)E * 256),
                "moe_eqb_bias: token bias");
    a = l.alpha;
  }
  moe::EqbWork w{l.hist, l.state, l.qraw};
  MOE_TRY_HIP(moe::launch_eqb(logits, a, N, E, K, key_bits, beta_out, quantile_out, w, st,
                              alpha == nullptr),
              "moe_eqb_bias");
  return ok();
}

static_assert(sizeof(moe_route_stats_t) == sizeof(moe::RouteStatsDev), "stats layout");
static_assert(offsetof(moe_route_stats_t, overlap) == offsetof(moe::RouteStatsDev, overlap),
              "stats layout");
static_assert(offsetof(moe_route_stats_t, max_load) == offsetof(moe::RouteStatsDev, max_load),
              "stats layout");

moe_status_t moe_route_stats(const int32_t* topk_ids, const int32_t* topk_ids_unbiased,
                             const float* margin, int64_t N, int32_t E, int32_t K, float tau,
                             int32_t* counts, moe_route_stats_t* stats, void* stream) {
  moe_status_t s = check_route_shape(N, E, K);
  if (s != MOE_OK) return s;
  if (!topk_ids || !counts || !stats)
    return fail(MOE_ERR_INVALID_ARGUMENT, "topk_ids, counts and stats are required");
  const void* p4[] = {topk_ids, topk_ids_unbiased, margin, counts};
  for (const void* q : p4)
    if (q && !aligned(q, 4)) return fail(MOE_ERR_INVALID_ARGUMENT, "pointer not 4-byte aligned");
  if (!aligned(stats, 8)) return fail(MOE_ERR_INVALID_ARGUMENT, "stats not 8-byte aligned");
  MOE_TRY_HIP(moe::launch_route_stats(topk_ids, topk_ids_unbiased, margin, N, E, K, tau, counts,
                                      reinterpret_cast<moe::RouteStatsDev*>(stats),
                                      (hipStream_t)stream),
              "moe_route_stats");
  return ok();
}

size_t moe_lei_workspace_bytes(int32_t E) {
  if (E < 2 || E > MOE_MAX_E) return 0;
  Carver c(nullptr);
  c.take<int32_t>((size_t)E);
  c.take<float>((size_t)E);
  return c.off;
}

moe_status_t moe_lei_backward(const float* logits, const int32_t* topk_ids,
                              const float* grad_scores, int64_t N, int32_t E, int32_t K,
                              float lam, float tau, float* grad_scores_out,
                              float* grad_logits_out, float* injection_out, void* workspace,
                              size_t workspace_bytes, void* stream) {
  moe_status_t s = check_route_shape(N, E, K);
  if (s != MOE_OK) return s;
  if (!topk_ids) return fail(MOE_ERR_INVALID_ARGUMENT, "topk_ids is required");
  if (!grad_scores_out && !grad_logits_out)
    return fail(MOE_ERR_INVALID_ARGUMENT, "grad_scores_out or grad_logits_out is required");
  if (grad_logits_out && !logits)
    return fail(MOE_ERR_INVALID_ARGUMENT, "logits are required for grad_logits_out");
  if (!(tau > 0.0f) || !std::isfinite(tau) || !std::isfinite(lam))
    return fail(MOE_ERR_INVALID_ARGUMENT, "lam must be finite and tau finite and > 0");
  const void* p4[] = {logits, topk_ids, grad_scores, grad_scores_out, grad_logits_out,
                      injection_out};
  for (const void* q : p4)
    if (q && !aligned(q, 4)) return fail(MOE_ERR_INVALID_ARGUMENT, "pointer not 4-byte aligned");
  if (grad_logits_out && (grad_logits_out == grad_scores || grad_logits_out == logits))
    return fail(MOE_ERR_INVALID_ARGUMENT, "grad_logits_out must not alias an input");
  const size_t need = moe_lei_workspace_bytes(E);
  if (!workspace || !aligned(workspace, kAlign))
    return fail(MOE_ERR_INVALID_ARGUMENT, "workspace must be non-NULL and 256-byte aligned");
  if (workspace_bytes < need)
    return fail(MOE_ERR_WORKSPACE_TOO_SMALL, "workspace %zu < required %zu", workspace_bytes, need);
  Carver c(workspace);
  int32_t* counts = c.take<int32_t>((size_t)E);
  float* inj = c.take<float>((size_t)E);
  MOE_TRY_HIP(moe::launch_lei(logits, topk_ids, grad_scores, N, E, K, lam, tau, grad_scores_out,
                              grad_logits_out, injection_out, counts, inj, (hipStream_t)stream),
              "moe_lei_backward");
  return ok();
}

// ---- exact quantile update over a batch that arrives in several parts
// State: histograms, selection state, raw quantiles.
static moe::EqbWork carve_eqb_state(Carver& c, int E, int key_bits) {
  moe::EqbWork w;
  w.hist = c.take<uint32_t>(moe::eqb_hist_bytes(E, key_bits) / 4);
  w.state = c.take<uint32_t>(moe::eqb_state_bytes(E) / 4);
  w.qraw = c.take<float>((size_t)E);
  return w;
}

static moe_status_t check_eqb_state(int32_t E, int32_t key_bits, const void* state,
                                    size_t state_bytes) {
  if (E < 2 || E > MOE_MAX_E) return fail(MOE_ERR_UNSUPPORTED_SHAPE, "E=%d outside [2, %d]", E, MOE_MAX_E);
  if (key_bits != 16 && key_bits != 32)
    return fail(MOE_ERR_INVALID_ARGUMENT, "key_bits=%d must be 16 or 32", key_bits);
  if (!state || !aligned(state, kAlign))
    return fail(MOE_ERR_INVALID_ARGUMENT, "state must be non-NULL and 256-byte aligned");
  const size_t need = moe_eqb_state_bytes(E, key_bits);
  if (state_bytes < need)
    return fail(MOE_ERR_WORKSPACE_TOO_SMALL, "state %zu < required %zu", state_bytes, need);
  return MOE_OK;
}

size_t moe_eqb_state_bytes(int32_t E, int32_t key_bits) {
  if (E < 2 || E > MOE_MAX_E || (key_bits != 16 && key_bits != 32)) return 0;
  Carver c(nullptr);
  carve_eqb_state(c, E, key_bits);
  return c.off;
}

moe_status_t moe_eqb_begin(int32_t E, int32_t key_bits, void* state, size_t state_bytes,
                           void* stream) {
  moe_status_t s = check_eqb_state(E, key_bits, state, state_bytes);
  if (s != MOE_OK) return s;
  Carver c(state);
  const moe::EqbWork w = carve_eqb_state(c, E, key_bits);
  MOE_TRY_HIP(moe::launch_fill_u32(w.hist, 0u, moe::eqb_hist_bytes(E, key_bits) / 4,
                                   (hipStream_t)stream), "moe_eqb_begin");
  return ok();
}

moe_status_t moe_eqb_accumulate(int32_t pass, const float* logits, const float* alpha,
                                int64_t N, int32_t E, int32_t key_bits, void* state,
                                size_t state_bytes, void* stream) {
  moe_status_t s = check_eqb_state(E, key_bits, state, state_bytes);
  if (s != MOE_OK) return s;
  if (N < 1 || N > (int64_t(1) << 24)) return fail(MOE_ERR_UNSUPPORTED_SHAPE, "N=%lld outside [1, 2^24]", (long long)N);
  if (pass < 0 || pass >= key_bits / 8)
    return fail(MOE_ERR_INVALID_ARGUMENT, "pass=%d outside [0, %d)", pass, key_bits / 8);
  if (!logits || !alpha) return fail(MOE_ERR_INVALID_ARGUMENT, "logits and alpha are required");
  if (!aligned(logits, 4) || !aligned(alpha, 4))
    return fail(MOE_ERR_INVALID_ARGUMENT, "pointer not 4-byte aligned");
  Carver c(state);
  const moe::EqbWork w = carve_eqb_state(c, E, key_bits);
  MOE_TRY_HIP(moe::launch_eqb_hist(logits, alpha, N, E, key_bits, pass, w.state,
                                   w.hist + (size_t)pass * E * 256, (hipStream_t)stream),
              "moe_eqb_accumulate");
  return ok();
}

moe_status_t moe_eqb_select(int32_t pass, int64_t n_total, int32_t E, int32_t K,
                            int32_t key_bits, float* beta_out, float* quantile_out,
                            void* state, size_t state_bytes, void* stream) {
  moe_status_t s = check_eqb_state(E, key_bits, state, state_bytes);
  if (s != MOE_OK) return s;
  s = check_route_shape(n_total, E, K);
  if (s != MOE_OK) return s;
  if (pass < 0 || pass >= key_bits / 8)
    return fail(MOE_ERR_INVALID_ARGUMENT, "pass=%d outside [0, %d)", pass, key_bits / 8);
  const bool last = pass == key_bits / 8 - 1;
  if (last && !beta_out) return fail(MOE_ERR_INVALID_ARGUMENT, "beta_out is required at the last pass");
  if ((beta_out && !aligned(beta_out, 4)) || (quantile_out && !aligned(quantile_out, 4)))
    return fail(MOE_ERR_INVALID_ARGUMENT, "pointer not 4-byte aligned");
  Carver c(state);
  const moe::EqbWork w = carve_eqb_state(c, E, key_bits);
  MOE_TRY_HIP(moe::launch_eqb_scan(w, E, K, key_bits, pass, n_total, last ? beta_out : nullptr,
                                   last ? quantile_out : nullptr, (hipStream_t)stream),
              "moe_eqb_select");
  return ok();
}

size_t moe_forward_workspace_bytes(const moe_problem_t* p) {
  if (check_problem(p) != MOE_OK) return 0;
  return carve_forward(nullptr, *p).bytes;
}

size_t moe_forward_fp8_workspace_bytes(const moe_problem_t* p) {
  if (check_problem_fp8(p) != MOE_OK) return 0;
  return carve_forward(nullptr, *p, true).bytes;
}

moe_status_t moe_forward(const moe_problem_t* p, const moe_weights_t* w, const uint16_t* x,
                         const float* beta_in, uint16_t* y, moe_aux_t* aux, void* workspace,
                         size_t workspace_bytes, void* stream) {
  return moe::forward_bf16(p, w, x, beta_in, y, aux, workspace, workspace_bytes, stream, false);
}

}  // extern "C"

// moe_forward's checks and launches; with in_order the call neither creates
// nor uses the side stream (the shared expert runs on `stream`) and records no
// stage timing.
moe_status_t moe::forward_bf16(const moe_problem_t* p, const moe_weights_t* w, const uint16_t* x,
                               const float* beta_in, uint16_t* y, moe_aux_t* aux,
                               void* workspace, size_t workspace_bytes, void* stream,
                               bool in_order) {
  moe_status_t s = check_problem(p);
  if (s != MOE_OK) return s;
  if (!w || !x || !y) return fail(MOE_ERR_INVALID_ARGUMENT, "weights, x and y are required");
  if (!w->w_gate || !w->w_up || !w->w_down)
    return fail(MOE_ERR_INVALID_ARGUMENT, "routed expert weights are required");
  if (p->n_shared == 1 && (!w->ws_gate || !w->ws_up || !w->ws_down))
    return fail(MOE_ERR_INVALID_ARGUMENT, "shared expert weights are required");
  const void* p16[] = {w->w_router, w->w_gate, w->w_up, w->w_down, w->ws_gate, w->ws_up, w->ws_down};
  for (const void* q : p16)
    if (q && !aligned(q, 16)) return fail(MOE_ERR_INVALID_ARGUMENT, "bf16 buffers must be 16-byte aligned");
  Experts ex;
  ex.w_router = w->w_router;
  ex.b = w;
  ex.in_order = in_order;
  return forward_impl(p, ex, x, beta_in, y, aux, workspace, workspace_bytes, stream);
}

moe_status_t moe::set_error(moe_status_t s, const char* msg) { return fail(s, "%s", msg); }

extern "C" {

moe_status_t moe_forward_fp8(const moe_problem_t* p, const moe_fp8_weights_t* w,
                             const uint16_t* x, const float* beta_in, uint16_t* y,
                             moe_aux_t* aux, void* workspace, size_t workspace_bytes,
                             void* stream) {
  moe_status_t s = check_problem_fp8(p);
  if (s != MOE_OK) return s;
  if (!w || !x || !y) return fail(MOE_ERR_INVALID_ARGUMENT, "weights, x and y are required");
  if (!w->w_gate || !w->w_up || !w->w_down || !w->s_gate || !w->s_up || !w->s_down)
    return fail(MOE_ERR_INVALID_ARGUMENT, "routed expert codes and scales are required");
  if (p->n_shared == 1 && (!w->ws_gate || !w->ws_up || !w->ws_down || !w->ss_gate ||
                           !w->ss_up || !w->ss_down))
    return fail(MOE_ERR_INVALID_ARGUMENT, "shared expert codes and scales are required");
  const void* p16[] = {w->w_router, w->w_gate, w->w_up, w->w_down, w->ws_gate, w->ws_up, w->ws_down};
  for (const void* q : p16)
    if (q && !aligned(q, 16)) return fail(MOE_ERR_INVALID_ARGUMENT, "weight buffers must be 16-byte aligned");
  const void* p4[] = {w->s_gate, w->s_up, w->s_down, w->ss_gate, w->ss_up, w->ss_down};
  for (const void* q : p4)
    if (q && !aligned(q, 4)) return fail(MOE_ERR_INVALID_ARGUMENT, "scale buffers must be 4-byte aligned");
  Experts ex;
  ex.fp8 = true;
  ex.w_router = w->w_router;
  ex.q = w;
  return forward_impl(p, ex, x, beta_in, y, aux, workspace, workspace_bytes, stream);
}

moe_status_t moe_fp8_quantize_blocks(const uint16_t* w, int64_t count, int32_t rows,
                                     int32_t cols, uint8_t* codes, float* scales, void* stream) {
  if (count < 0 || count > 65535 || rows < 1 || rows > 65536 || cols < 1 || cols > 65536)
    return fail(MOE_ERR_UNSUPPORTED_SHAPE,
                "count=%lld rows=%d cols=%d: need 0 <= count <= 65535, 1 <= rows, cols <= 65536",
                (long long)count, rows, cols);
  if (count == 0) return ok();
  if (!w || !codes || !scales) return fail(MOE_ERR_INVALID_ARGUMENT, "w, codes and scales are required");
  if (!aligned(w, 2) || !aligned(scales, 4)) return fail(MOE_ERR_INVALID_ARGUMENT, "misaligned buffer");
  MOE_TRY_HIP(moe::launch_quant_blocks(w, count, rows, cols, codes, scales, (hipStream_t)stream),
              "moe_fp8_quantize_blocks");
  return ok();
}

moe_status_t moe_pack_gateup_weights(const uint16_t* w, int64_t count, int32_t rows,
                                     int32_t cols, uint16_t* out, void* stream) {
  if (count < 0 || count > 65535 || rows < 1 || rows > 65536 || cols < 64 || cols > 65536 ||
      cols % 64)
    return fail(MOE_ERR_UNSUPPORTED_SHAPE,
                "count=%lld rows=%d cols=%d: need 0 <= count <= 65535, 1 <= rows <= 65536 and "
                "cols a multiple of 64 in [64, 65536]",
                (long long)count, rows, cols);
  if (count == 0) return ok();
  if (!w || !out) return fail(MOE_ERR_INVALID_ARGUMENT, "w and out are required");
  if (!aligned(w, 16) || !aligned(out, 16))
    return fail(MOE_ERR_INVALID_ARGUMENT, "w and out must be 16-byte aligned");
  const size_t bytes = (size_t)count * (size_t)rows * (size_t)cols * 2u;
  const char* a0 = reinterpret_cast<const char*>(w);
  const char* b0 = reinterpret_cast<const char*>(out);
  if (a0 < b0 + bytes && b0 < a0 + bytes)
    return fail(MOE_ERR_INVALID_ARGUMENT, "out must not overlap w");
  MOE_TRY_HIP(moe::launch_pack_kblocks(w, count, rows, cols, out, (hipStream_t)stream),
              "moe_pack_gateup_weights");
  return ok();
}

moe_status_t moe_fp8_quantize_rows(const uint16_t* x, int64_t n, int32_t cols, uint8_t* codes,
                                   float* scales, void* stream) {
  if (n < 0 || n > (int64_t(1) << 27) || cols < 128 || cols > 65536 || cols % 128)
    return fail(MOE_ERR_UNSUPPORTED_SHAPE,
                "n=%lld cols=%d: need 0 <= n <= 2^27 and cols a multiple of 128 in [128, 65536]",
                (long long)n, cols);
  if (n == 0) return ok();
  if (!x || !codes || !scales) return fail(MOE_ERR_INVALID_ARGUMENT, "x, codes and scales are required");
  if (!aligned(x, 4) || !aligned(codes, 2) || !aligned(scales, 4))
    return fail(MOE_ERR_INVALID_ARGUMENT, "misaligned buffer");
  MOE_TRY_HIP(moe::launch_quant_rows(x, n, cols, codes, scales, (hipStream_t)stream),
              "moe_fp8_quantize_rows");
  return ok();
}

}  // extern "C"
