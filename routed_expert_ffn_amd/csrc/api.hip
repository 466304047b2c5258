// C ABI of libmoe.so (declared and documented in include/moe.h): argument
// validation, workspace carve-up and the launch sequence on the caller's
// stream (with one side stream for the shared experts).
// Nothing here allocates device memory, frees, synchronises or reads device
// memory, so every entry point can be captured in a HIP graph.
#include <stdarg.h>
#include <stdio.h>

#include <mutex>
#include <vector>

#include "internal.h"

namespace {

// Work that does not depend on the routing (the shared experts) runs on a
// second stream of the library, forked from the caller's stream after what
// the caller enqueued before and joined back before its result is read.  At
// decode sizes it is an HBM-bound GEMV and the routing is latency-bound, so
// the two overlap; the join comes before the combine, long after the branch
// has finished, so its latency is off the critical path.  Graph capture
// records the fork and the join as dependencies.  The stream and its two
// events are created, per device, by the first such call whose stream is not
// being captured (creation is not enqueued work); until then, and if creation
// fails, the branch runs on the caller's stream.  One lock per process is held
// from fork to join, so calls from several host threads use the events one at
// a time.
constexpr int SIDE_MAX_DEVICES = 64;
struct SideStream {
  hipStream_t s = nullptr;
  hipEvent_t fork = nullptr, join = nullptr;
};
std::mutex g_side_mu;
SideStream g_side[SIDE_MAX_DEVICES];

constexpr int SHARED_AFTER_ROUTE_T = 1024;

class SideBranch {
 public:
  explicit SideBranch(hipStream_t main) : main_(main), lk_(g_side_mu) {
    // the branch's kernels run on the side stream's device: use it only when
    // the caller's stream belongs to the current device
    int dev = -1;
    hipDevice_t sdev = -1;
    if (hipGetDevice(&dev) != hipSuccess || hipStreamGetDevice(main, &sdev) != hipSuccess || sdev != dev || dev < 0 ||
        dev >= SIDE_MAX_DEVICES) {
      (void)hipGetLastError();
      return;
    }
    SideStream& d = g_side[dev];
    if (!d.s && !create(d, main)) return;
    if (hipEventRecord(d.fork, main) != hipSuccess || hipStreamWaitEvent(d.s, d.fork, 0) != hipSuccess) {
      (void)hipGetLastError();
      return;
    }
    side_ = &d;
  }
  ~SideBranch() { (void)join(); }
  hipStream_t stream() const { return side_ ? side_->s : main_; }
  // the caller's stream waits for everything enqueued on the branch
  hipError_t join() {
    if (!side_) return hipSuccess;
    SideStream* d = side_;
    side_ = nullptr;
    hipError_t e = hipEventRecord(d->join, d->s);
    if (e == hipSuccess) e = hipStreamWaitEvent(main_, d->join, 0);
    return e;
  }

 private:
  static bool create(SideStream& d, hipStream_t main) {
    hipStreamCaptureStatus st = hipStreamCaptureStatusNone;
    if (hipStreamIsCapturing(main, &st) != hipSuccess || st != hipStreamCaptureStatusNone) {
      (void)hipGetLastError();
      return false;
    }
    SideStream n;
    const bool ok = hipStreamCreateWithFlags(&n.s, hipStreamNonBlocking) == hipSuccess &&
                    hipEventCreateWithFlags(&n.fork, hipEventDisableTiming) == hipSuccess &&
                    hipEventCreateWithFlags(&n.join, hipEventDisableTiming) == hipSuccess;
    if (!ok) {
      (void)hipGetLastError();
      if (n.join) (void)hipEventDestroy(n.join);
      if (n.fork) (void)hipEventDestroy(n.fork);
      if (n.s) (void)hipStreamDestroy(n.s);
      return false;
    }
    d = n;
    return true;
  }
  hipStream_t main_;
  std::lock_guard<std::mutex> lk_;
  SideStream* side_ = nullptr;
};

thread_local char g_err[512] = "";

moe_status fail(moe_status s, const char* fmt, ...) {
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(g_err, sizeof g_err, fmt, ap);
  va_end(ap);
  return s;
}

moe_status hip_fail(hipError_t e, const char* what) {
  return fail(MOE_ERR_HIP, "%s: %s", what, hipGetErrorString(e));
}

bool aligned16(const void* p) { return ((uintptr_t)p & 15u) == 0; }

struct Prof {
  int kernel = -1;
  std::vector<hipEvent_t> events;  // 2 per launch
  int used = 0;
  void release() {
    for (hipEvent_t e : events) (void)hipEventDestroy(e);
    events.clear();
    used = 0;
    kernel = -1;
  }
};
thread_local Prof g_prof;

// Routing (the router, top-k) needs E a multiple of 8 with at least k
// experts; the permutation of given ids and the expert pass take any id
// space of 1 .. 1024 experts (router = false), e.g. one device's experts.
moe_status check_dims(const moe_dims& d, bool router = true) {
  if (d.T < 0) return fail(MOE_ERR_SHAPE, "T = %d is negative", d.T);
  if (d.H <= 0 || d.H % 256) return fail(MOE_ERR_SHAPE, "H = %d must be a positive multiple of 256", d.H);
  if (d.I <= 0 || d.I % 256) return fail(MOE_ERR_SHAPE, "I = %d must be a positive multiple of 256", d.I);
  if (d.k < 1 || d.k > 64) return fail(MOE_ERR_SHAPE, "k = %d must be in [1, 64]", d.k);
  if (router && (d.E < d.k || d.E > 1024 || d.E % 8))
    return fail(MOE_ERR_SHAPE, "E = %d must be a multiple of 8 in [k, 1024]", d.E);
  if (!router && (d.E < 1 || d.E > 1024)) return fail(MOE_ERR_SHAPE, "E = %d must be in [1, 1024]", d.E);
  if ((long long)d.T * d.k >= (1LL << 31)) return fail(MOE_ERR_SHAPE, "T*k = %lld is too large", (long long)d.T * d.k);
  // grids take one row per token (at most 65535), and the large-batch GEMMs
  // address token rows (2 T H bytes of x, 2 T k I of h) with 32-bit offsets
  if (d.T > 65535) return fail(MOE_ERR_SHAPE, "T = %d exceeds 65535 tokens per call", d.T);
  const long long ki = (long long)d.k * d.I, wide = d.H > ki ? d.H : ki;
  if ((long long)d.T * wide >= (1LL << 31))
    return fail(MOE_ERR_SHAPE, "T * max(H, k*I) = %lld must be below 2^31", (long long)d.T * wide);
  return MOE_OK;
}

size_t align256(size_t b) { return (b + 255) & ~(size_t)255; }

// Workspace regions (byte offsets, 256-byte aligned).  moe_layer uses all of
// them; moe_route and moe_expert_ffn use subsets of the same layout.
struct Layout {
  size_t part, logits, ids, w, lids, masks, counts, base, offsets, sorted, pos, active, nact, mtiles, nmt, x16, h,
      rows, total;
};

Layout layout(const moe_dims& d) {
  Layout L;
  size_t o = 0;
  auto take = [&](size_t bytes) {
    size_t r = o;
    o += align256(bytes);
    return r;
  };
  const size_t T = (size_t)d.T, H = (size_t)d.H, I = (size_t)d.I, E = (size_t)d.E, P = T * (size_t)d.k;
  const size_t S = (size_t)moe::router_plan(d.T, d.H, d.E).slabs, nb = (size_t)moe::perm_blocks(d.T);
  L.part = take(S * T * E * 4);
  L.logits = take(T * E * 4);
  L.ids = take(P * 4);
  L.w = take(P * 4);
  L.lids = take(P * 4);
  L.masks = take(nb * E * 8);
  L.counts = take(nb * E * 4);
  L.base = take(nb * E * 4);
  L.offsets = take((E + 1) * 4);
  L.sorted = take(P * 4);
  L.pos = take(P * 4);
  L.active = take(E * 4);
  L.nact = take(4);
  L.mtiles = take((size_t)moe::max_mtiles(d) * 4);
  L.nmt = take(4);
  L.x16 = take((T + 1) * H * 2);  // row T: zeros (the large-tile GEMMs' padding rows)
  L.h = take((P + 1) * I * 2);    // row P: zeros
  L.rows = take(P * H * 4);
  L.total = o;
  return L;
}

// moe_latent_layer: moe_layer's regions for the latent width, then the
// router's partials over the hidden width, the projections' partials, the
// latent z and the combined latent output.
struct LatentLayout {
  Layout base;
  size_t rpart, ppart, z, ylat, total;
};

LatentLayout latent_layout(const moe_dims& d, int Hm) {
  LatentLayout LL;
  LL.base = layout(d);
  size_t o = LL.base.total;
  auto take = [&](size_t bytes) {
    size_t r = o;
    o += align256(bytes);
    return r;
  };
  const size_t T = (size_t)d.T, H = (size_t)d.H, E = (size_t)d.E, M = (size_t)Hm;
  const moe::RouterPlan rr = moe::router_plan(d.T, Hm, d.E), rd = moe::router_plan(d.T, Hm, d.H),
                        ru = moe::router_plan(d.T, d.H, Hm);
  LL.rpart = take((size_t)rr.slabs * T * E * 4);
  // a tiled projection of one slab writes its output directly
  const size_t down = rd.tiled && rd.slabs == 1 ? 0 : (size_t)rd.slabs * T * H * 4;
  const size_t up = ru.tiled && ru.slabs == 1 ? 0 : (size_t)ru.slabs * T * M * 4;
  LL.ppart = take(down > up ? down : up);
  LL.z = take(T * H * 2);
  LL.ylat = take(T * H * 2);
  LL.total = o;
  return LL;
}

// moe_layer_shared: moe_layer's regions, then the shared experts' gate/up
// partials, their hidden layer and their down partials.
struct SharedLayout {
  Layout base;
  size_t gupart, h, dpart, total;
  int gu_slabs, d_slabs;
};

SharedLayout shared_layout(const moe_dims& d, const moe_shared& sh) {
  SharedLayout SL;
  SL.base = layout(d);
  size_t o = SL.base.total;
  auto take = [&](size_t bytes) {
    size_t r = o;
    o += align256(bytes);
    return r;
  };
  const int width = sh.count * sh.I;
  const size_t T = (size_t)d.T;
  const moe::RouterPlan gu = moe::router_plan(d.T, d.H, 2 * width), dn = moe::router_plan(d.T, width, d.H);
  SL.gu_slabs = gu.slabs;
  SL.d_slabs = dn.slabs;
  SL.gupart = take((size_t)SL.gu_slabs * T * 2 * width * 4);
  SL.h = take(T * width * 2);
  SL.dpart = take((size_t)SL.d_slabs * T * d.H * 4);
  SL.total = o;
  return SL;
}

moe_status check_shared(const moe_shared* sh) {
  if (!sh) return fail(MOE_ERR_ARG, "shared is NULL");
  if (sh->count < 1 || sh->count > 64) return fail(MOE_ERR_SHAPE, "shared count = %d must be in [1, 64]", sh->count);
  if (sh->I <= 0 || sh->I % 256) return fail(MOE_ERR_SHAPE, "shared I = %d must be a positive multiple of 256", sh->I);
  return MOE_OK;
}

moe_status check_latent_width(int Hm) {
  if (Hm <= 0 || Hm % 256) return fail(MOE_ERR_SHAPE, "H_model = %d must be a positive multiple of 256", Hm);
  return MOE_OK;
}

template <class T>
T* at(void* ws, size_t off) {
  return reinterpret_cast<T*>(static_cast<char*>(ws) + off);
}

moe_status check_ws(const moe_dims& d, void* ws, size_t ws_bytes) {
  const size_t need = layout(d).total;
  if (!ws) return fail(MOE_ERR_ARG, "workspace is NULL");
  if (!aligned16(ws)) return fail(MOE_ERR_ALIGN, "workspace is not 16-byte aligned");
  if (ws_bytes < need) return fail(MOE_ERR_WORKSPACE, "workspace has %zu bytes, needs %zu", ws_bytes, need);
  return MOE_OK;
}

moe_status check_ptr(const void* p, const char* name, bool required = true) {
  if (!p) return required ? fail(MOE_ERR_ARG, "%s is NULL", name) : MOE_OK;
  if (!aligned16(p)) return fail(MOE_ERR_ALIGN, "%s is not 16-byte aligned", name);
  return MOE_OK;
}

moe_status check_experts(const moe_experts* w) {
  if (!w) return fail(MOE_ERR_ARG, "experts struct is NULL");
  if (w->format != MOE_FMT_NVFP4 && w->format != MOE_FMT_MXFP4)
    return fail(MOE_ERR_ARG, "experts format = %d is not a moe_weight_format", (int)w->format);
  const moe_nvfp4* m[3] = {&w->gate, &w->up, &w->down};
  const char* names[3] = {"gate", "up", "down"};
  for (int i = 0; i < 3; i++) {
    if (!m[i]->q || !m[i]->sf || !m[i]->gs) return fail(MOE_ERR_ARG, "%s weights have a NULL pointer", names[i]);
    if (!aligned16(m[i]->q) || !aligned16(m[i]->sf))
      return fail(MOE_ERR_ALIGN, "%s codes or scales are not 16-byte aligned", names[i]);
    if ((uintptr_t)m[i]->gs & 3u) return fail(MOE_ERR_ALIGN, "%s per-tensor scales are not 4-byte aligned", names[i]);
  }
  return MOE_OK;
}

#define TRY(expr)                       \
  do {                                  \
    moe_status _s = (expr);             \
    if (_s != MOE_OK) return _s;        \
  } while (0)

#define LAUNCH(kernel_id, stream, call, what)    \
  do {                                           \
    moe::prof_before(kernel_id, stream);         \
    hipError_t _e = (call);                      \
    if (_e != hipSuccess) return hip_fail(_e, what); \
    moe::prof_after(kernel_id, stream);          \
  } while (0)

// Enqueue routing; logits are an input when x == NULL.  When x16 is given,
// the router also writes the fp16 copy of x the FFN reads.
moe_status enqueue_route(const moe_dims& d, const void* x, const void* wr, const float* bias, float* logits,
                         int32_t* ids, float* w, int32_t* offsets, int32_t* sorted, int32_t* pos, void* ws,
                         f16* x16, hipStream_t s) {
  const Layout L = layout(d);
  const moe::RouterPlan rp = moe::router_plan(d.T, d.H, d.E);
  if (x)
    LAUNCH(MOE_KERNEL_ROUTER, s,
           moe::launch_router(static_cast<const uint16_t*>(x), static_cast<const uint16_t*>(wr),
                              at<float>(ws, L.part), d.T, d.H, d.E, rp, s, x16),
           "router");
  if (moe::route_fused(d.T)) {  // top-k and permutation in one launch, timed as top-k
    LAUNCH(MOE_KERNEL_TOPK, s,
           moe::launch_route_small(x ? at<float>(ws, L.part) : nullptr, rp.slabs, x ? bias : nullptr, logits, d.T,
                                   d.E, d.k, ids, w, offsets, sorted, pos, at<int32_t>(ws, L.active),
                                   at<int32_t>(ws, L.nact), s),
           "route");
    return MOE_OK;
  }
  LAUNCH(MOE_KERNEL_TOPK, s,
         moe::launch_topk(x ? at<float>(ws, L.part) : nullptr, rp.slabs, x ? bias : nullptr, logits, d.T, d.E, d.k,
                          ids, w, s),
         "top-k");
  LAUNCH(MOE_KERNEL_PERMUTE, s,
         moe::launch_permute(ids, d.T, d.E, d.k, at<uint64_t>(ws, L.masks), at<int32_t>(ws, L.counts),
                             at<int32_t>(ws, L.base), offsets, sorted, pos, at<int32_t>(ws, L.active),
                             at<int32_t>(ws, L.nact), at<int32_t>(ws, L.mtiles), at<int32_t>(ws, L.nmt), s),
         "permute");
  return MOE_OK;
}

// Enqueue the two grouped GEMMs (x16, the active list and the permutation
// are already in place).
moe_status enqueue_ffn(const moe_dims& d, const int32_t* offsets, const int32_t* sorted, const moe_experts* w,
                       float* rows, void* ws, hipStream_t s, int e_base = 0, f16* rows16 = nullptr,
                       const float* pair_w = nullptr) {
  const Layout L = layout(d);
  moe::FfnArgs a;
  a.T = d.T;
  a.H = d.H;
  a.I = d.I;
  a.E = d.E;
  a.k = d.k;
  a.e_base = e_base;
  a.max_active = moe::max_active(d);
  a.x16 = at<f16>(ws, L.x16);
  a.offsets = offsets;
  a.sorted_pairs = sorted;
  a.active = at<int32_t>(ws, L.active);
  a.n_active = at<int32_t>(ws, L.nact);
  a.mtiles = at<int32_t>(ws, L.mtiles);
  a.n_mtiles = at<int32_t>(ws, L.nmt);
  a.max_mtiles = moe::max_mtiles(d);
  a.w = w;
  a.h = at<f16>(ws, L.h);
  a.rows = rows;
  a.rows16 = rows16;
  a.pair_w = pair_w;
  if (moe::pads_with_zero_rows(a))  // (a one-block kernel, outside the timing hooks)
    if (hipError_t e = moe::launch_zero_pad_rows(a, s); e != hipSuccess) return hip_fail(e, "zero rows");
  LAUNCH(MOE_KERNEL_GATEUP, s, moe::launch_gateup(a, s), "gate/up");
  LAUNCH(MOE_KERNEL_DOWN, s, moe::launch_down(a, s), "down");
  return MOE_OK;
}

moe_status expert_ffn_range(moe_dims d, int lo, int hi, const void* x, const int32_t* expert_offsets,
                            const int32_t* sorted_pairs, const moe_experts* w, float* rows, void* ws, size_t ws_bytes,
                            void* stream) {
  TRY(check_dims(d, false));
  if (d.T == 0) return MOE_OK;
  TRY(check_ptr(x, "x"));
  TRY(check_ptr(expert_offsets, "expert_offsets"));
  TRY(check_ptr(sorted_pairs, "sorted_pairs"));
  TRY(check_experts(w));
  TRY(check_ptr(rows, "rows"));
  TRY(check_ws(d, ws, ws_bytes));
  const Layout L = layout(d);
  hipStream_t s = (hipStream_t)stream;
  LAUNCH(MOE_KERNEL_CAST, s,
         moe::launch_active_list(expert_offsets, d.E, lo, hi, at<int32_t>(ws, L.active), at<int32_t>(ws, L.nact),
                                 at<int32_t>(ws, L.mtiles), at<int32_t>(ws, L.nmt), s),
         "active list");
  LAUNCH(MOE_KERNEL_CAST, s,
         moe::launch_cast(static_cast<const uint16_t*>(x), at<f16>(ws, L.x16), (long long)d.T * d.H, s), "cast");
  return enqueue_ffn(d, expert_offsets, sorted_pairs, w, rows, ws, s, lo);
}

moe_status check_share(const moe_dims& d, moe_expert_share sh) {
  if (sh.base < 0 || sh.count < 1 || sh.base > d.E - sh.count)
    return fail(MOE_ERR_SHAPE, "share [%d, %d + %d) is not a non-empty range of the %d experts", sh.base, sh.base,
                sh.count, d.E);
  return MOE_OK;
}


}  // namespace

void moe::prof_before(moe_kernel k, hipStream_t s) {
  if (g_prof.kernel == (int)k && 2 * g_prof.used < (int)g_prof.events.size())
    (void)hipEventRecord(g_prof.events[2 * g_prof.used], s);
}

void moe::prof_after(moe_kernel k, hipStream_t s) {
  if (g_prof.kernel == (int)k && 2 * g_prof.used < (int)g_prof.events.size()) {
    (void)hipEventRecord(g_prof.events[2 * g_prof.used + 1], s);
    g_prof.used++;
  }
}

extern "C" {

size_t moe_workspace_bytes(moe_dims d) {
  if (check_dims(d, false) != MOE_OK) return 0;
  return layout(d).total;
}

size_t moe_quantize_workspace_bytes(void) { return 256; }

static moe_status quantize_any(bool mx, const float* w, int64_t N, int64_t K, uint8_t* q, uint8_t* sf, float* gs, void* ws,
                               size_t ws_bytes, void* stream) {
  const int blk = mx ? 32 : 16;
  if (N < 1 || K < blk || K % blk)
    return fail(MOE_ERR_SHAPE, "N = %lld, K = %lld: need N >= 1 and K a multiple of %d", (long long)N, (long long)K,
                blk);
  TRY(check_ptr(w, "w"));
  TRY(check_ptr(q, "q"));
  if (!sf || !gs) return fail(MOE_ERR_ARG, "sf or gs is NULL");
  if ((uintptr_t)gs & 3u) return fail(MOE_ERR_ALIGN, "gs is not 4-byte aligned");
  if (!ws) return fail(MOE_ERR_ARG, "workspace is NULL");
  if ((uintptr_t)ws & 3u) return fail(MOE_ERR_ALIGN, "workspace is not 4-byte aligned");
  if (ws_bytes < moe_quantize_workspace_bytes())
    return fail(MOE_ERR_WORKSPACE, "workspace has %zu bytes, needs %zu", ws_bytes, moe_quantize_workspace_bytes());
  hipError_t e = mx ? moe::launch_quantize_mx(w, N, K, q, sf, gs, static_cast<uint32_t*>(ws), (hipStream_t)stream)
                    : moe::launch_quantize(w, N, K, q, sf, gs, static_cast<uint32_t*>(ws), (hipStream_t)stream);
  if (e != hipSuccess) return hip_fail(e, "quantize");
  return MOE_OK;
}

moe_status moe_quantize_nvfp4(const float* w, int64_t N, int64_t K, uint8_t* q, uint8_t* sf, float* gs, void* ws,
                              size_t ws_bytes, void* stream) {
  return quantize_any(false, w, N, K, q, sf, gs, ws, ws_bytes, stream);
}

moe_status moe_quantize_mxfp4(const float* w, int64_t N, int64_t K, uint8_t* q, uint8_t* sf, float* gs, void* ws,
                              size_t ws_bytes, void* stream) {
  return quantize_any(true, w, N, K, q, sf, gs, ws, ws_bytes, stream);
}

moe_status moe_route(moe_dims d, const void* x, const void* w_router, const float* bias, float* logits,
                     int32_t* topk_ids, float* topk_w, int32_t* expert_offsets, int32_t* sorted_pairs,
                     int32_t* pair_pos, void* ws, size_t ws_bytes, void* stream) {
  TRY(check_dims(d));
  if (d.T == 0) return MOE_OK;
  TRY(check_ptr(x, "x", false));
  if (x) TRY(check_ptr(w_router, "w_router"));
  TRY(check_ptr(bias, "bias", false));
  TRY(check_ptr(logits, "logits"));
  TRY(check_ptr(topk_ids, "topk_ids"));
  TRY(check_ptr(topk_w, "topk_w"));
  TRY(check_ptr(expert_offsets, "expert_offsets"));
  TRY(check_ptr(sorted_pairs, "sorted_pairs"));
  TRY(check_ptr(pair_pos, "pair_pos"));
  TRY(check_ws(d, ws, ws_bytes));
  return enqueue_route(d, x, w_router, bias, logits, topk_ids, topk_w, expert_offsets, sorted_pairs, pair_pos, ws,
                       nullptr, (hipStream_t)stream);
}

moe_status moe_expert_ffn(moe_dims d, const void* x, const int32_t* expert_offsets, const int32_t* sorted_pairs,
                          const moe_experts* w, float* rows, void* ws, size_t ws_bytes, void* stream) {
  return expert_ffn_range(d, 0, d.E, x, expert_offsets, sorted_pairs, w, rows, ws, ws_bytes, stream);
}

moe_status moe_expert_ffn_share(moe_dims d, moe_expert_share share, const void* x, const int32_t* expert_offsets,
                                const int32_t* sorted_pairs, const moe_experts* w, float* rows, void* ws,
                                size_t ws_bytes, void* stream) {
  TRY(check_dims(d));
  TRY(check_share(d, share));
  return expert_ffn_range(d, share.base, share.base + share.count, x, expert_offsets, sorted_pairs, w, rows, ws,
                          ws_bytes, stream);
}

moe_status moe_layer_share(moe_dims d, moe_expert_share share, const void* x, const void* w_router, const float* bias,
                           const moe_experts* w, float* y_partial, uint8_t* served, int32_t* topk_ids_out,
                           float* topk_w_out, void* ws, size_t ws_bytes, void* stream) {
  TRY(check_dims(d));
  TRY(check_share(d, share));
  if (d.T == 0) return MOE_OK;
  TRY(check_ptr(x, "x"));
  TRY(check_ptr(w_router, "w_router"));
  TRY(check_ptr(bias, "bias", false));
  TRY(check_experts(w));
  TRY(check_ptr(y_partial, "y_partial"));
  TRY(check_ptr(topk_ids_out, "topk_ids_out", false));
  TRY(check_ptr(topk_w_out, "topk_w_out", false));
  TRY(check_ws(d, ws, ws_bytes));
  const Layout L = layout(d);
  hipStream_t s = (hipStream_t)stream;
  const int lo = share.base, hi = share.base + share.count;
  int32_t* ids = topk_ids_out ? topk_ids_out : at<int32_t>(ws, L.ids);
  float* wts = topk_w_out ? topk_w_out : at<float>(ws, L.w);
  int32_t* offsets = at<int32_t>(ws, L.offsets);
  int32_t* sorted = at<int32_t>(ws, L.sorted);
  int32_t* pos = at<int32_t>(ws, L.pos);
  float* rows = at<float>(ws, L.rows);
  TRY(enqueue_route(d, x, w_router, bias, at<float>(ws, L.logits), ids, wts, offsets, sorted, pos, ws,
                    at<f16>(ws, L.x16), s));
  // the share's experts only: its active list and tile entries replace the routing's
  LAUNCH(MOE_KERNEL_PERMUTE, s,
         moe::launch_active_list(offsets, d.E, lo, hi, at<int32_t>(ws, L.active), at<int32_t>(ws, L.nact),
                                 at<int32_t>(ws, L.mtiles), at<int32_t>(ws, L.nmt), s),
         "active list");
  TRY(enqueue_ffn(d, offsets, sorted, w, rows, ws, s, lo));
  LAUNCH(MOE_KERNEL_COMBINE, s,
         moe::launch_combine_share(rows, pos, wts, ids, lo, hi, d.T, d.H, d.k, y_partial, served, s), "combine");
  return MOE_OK;
}

moe_status moe_permute(moe_dims d, const int32_t* topk_ids, int32_t* expert_offsets, int32_t* sorted_pairs,
                       int32_t* pair_pos, void* ws, size_t ws_bytes, void* stream) {
  TRY(check_dims(d, false));
  if (d.T == 0) return MOE_OK;
  TRY(check_ptr(topk_ids, "topk_ids"));
  TRY(check_ptr(expert_offsets, "expert_offsets"));
  TRY(check_ptr(sorted_pairs, "sorted_pairs"));
  TRY(check_ptr(pair_pos, "pair_pos"));
  TRY(check_ws(d, ws, ws_bytes));
  const Layout L = layout(d);
  hipStream_t s = (hipStream_t)stream;
  LAUNCH(MOE_KERNEL_PERMUTE, s,
         moe::launch_permute(topk_ids, d.T, d.E, d.k, at<uint64_t>(ws, L.masks), at<int32_t>(ws, L.counts),
                             at<int32_t>(ws, L.base), expert_offsets, sorted_pairs, pair_pos, at<int32_t>(ws, L.active),
                             at<int32_t>(ws, L.nact), at<int32_t>(ws, L.mtiles), at<int32_t>(ws, L.nmt), s),
         "permute");
  return MOE_OK;
}

moe_status moe_layer_mapped(moe_dims d, const int32_t* expert_map, int32_t n_local, const void* x,
                            const void* w_router, const float* bias, const moe_experts* w, float* y_partial,
                            uint8_t* served, int32_t* topk_ids_out, float* topk_w_out, int32_t* local_ids_out,
                            void* ws, size_t ws_bytes, void* stream) {
  TRY(check_dims(d));
  if (n_local < 1 || n_local > d.E) return fail(MOE_ERR_SHAPE, "n_local = %d must be in [1, E = %d]", n_local, d.E);
  if (d.T == 0) return MOE_OK;
  TRY(check_ptr(expert_map, "expert_map"));
  TRY(check_ptr(x, "x"));
  TRY(check_ptr(w_router, "w_router"));
  TRY(check_ptr(bias, "bias", false));
  TRY(check_experts(w));
  TRY(check_ptr(y_partial, "y_partial"));
  TRY(check_ptr(topk_ids_out, "topk_ids_out", false));
  TRY(check_ptr(topk_w_out, "topk_w_out", false));
  TRY(check_ptr(local_ids_out, "local_ids_out", false));
  TRY(check_ws(d, ws, ws_bytes));
  const Layout L = layout(d);
  hipStream_t s = (hipStream_t)stream;
  const int T = d.T, E = d.E, k = d.k;
  int32_t* ids = topk_ids_out ? topk_ids_out : at<int32_t>(ws, L.ids);
  float* wts = topk_w_out ? topk_w_out : at<float>(ws, L.w);
  int32_t* lids = local_ids_out ? local_ids_out : at<int32_t>(ws, L.lids);
  int32_t* offsets = at<int32_t>(ws, L.offsets);
  int32_t* sorted = at<int32_t>(ws, L.sorted);
  int32_t* pos = at<int32_t>(ws, L.pos);
  float* rows = at<float>(ws, L.rows);
  // routing over all E experts (the router also writes the fp16 copy of x);
  // the single-launch routing of small batches also permutes over all E,
  // which the local permutation below replaces
  const moe::RouterPlan rp = moe::router_plan(T, d.H, E);
  LAUNCH(MOE_KERNEL_ROUTER, s,
         moe::launch_router(static_cast<const uint16_t*>(x), static_cast<const uint16_t*>(w_router),
                            at<float>(ws, L.part), T, d.H, E, rp, s, at<f16>(ws, L.x16)),
         "router");
  if (moe::route_fused(T))
    LAUNCH(MOE_KERNEL_TOPK, s,
           moe::launch_route_small(at<float>(ws, L.part), rp.slabs, bias, at<float>(ws, L.logits), T, E, k, ids, wts,
                                   offsets, sorted, pos, at<int32_t>(ws, L.active), at<int32_t>(ws, L.nact), s),
           "route");
  else
    LAUNCH(MOE_KERNEL_TOPK, s,
           moe::launch_topk(at<float>(ws, L.part), rp.slabs, bias, at<float>(ws, L.logits), T, E, k, ids, wts, s),
           "top-k");
  // the mask on the chosen ids: global ids to slots of this store, -1 elsewhere
  LAUNCH(MOE_KERNEL_PERMUTE, s, moe::launch_remap_ids(ids, expert_map, E, n_local, (long long)T * k, lids, s),
         "remap");
  LAUNCH(MOE_KERNEL_PERMUTE, s,
         moe::launch_permute(lids, T, n_local, k, at<uint64_t>(ws, L.masks), at<int32_t>(ws, L.counts),
                             at<int32_t>(ws, L.base), offsets, sorted, pos, at<int32_t>(ws, L.active),
                             at<int32_t>(ws, L.nact), at<int32_t>(ws, L.mtiles), at<int32_t>(ws, L.nmt), s),
         "permute");
  TRY(enqueue_ffn(d, offsets, sorted, w, rows, ws, s, 0));
  LAUNCH(MOE_KERNEL_COMBINE, s,
         moe::launch_combine_share(rows, pos, wts, lids, 0, n_local, T, d.H, k, y_partial, served, s), "combine");
  return MOE_OK;
}

}  // extern "C"

namespace {

moe_status check_layer_args(const moe_dims& d, const void* x, const void* w_router, const float* bias,
                            const moe_experts* w, void* y, int32_t* topk_ids_out, float* topk_w_out) {
  TRY(check_ptr(x, "x"));
  TRY(check_ptr(w_router, "w_router"));
  TRY(check_ptr(bias, "bias", false));
  TRY(check_experts(w));
  TRY(check_ptr(y, "y"));
  TRY(check_ptr(topk_ids_out, "topk_ids_out", false));
  TRY(check_ptr(topk_w_out, "topk_w_out", false));
  return MOE_OK;
}

// moe_layer's launches on a validated call; ws holds at least the regions
// up to and including the fp16 rows (layout_rows16_bytes).
moe_status enqueue_layer(const moe_dims& d, const void* x, const void* w_router, const float* bias,
                         const moe_experts* w, void* y, int32_t* topk_ids_out, float* topk_w_out, void* ws,
                         hipStream_t s) {
  const Layout L = layout(d);
  int32_t* ids = topk_ids_out ? topk_ids_out : at<int32_t>(ws, L.ids);
  float* wts = topk_w_out ? topk_w_out : at<float>(ws, L.w);
  int32_t* offsets = at<int32_t>(ws, L.offsets);
  int32_t* sorted = at<int32_t>(ws, L.sorted);
  int32_t* pos = at<int32_t>(ws, L.pos);
  float* rows = at<float>(ws, L.rows);
  TRY(enqueue_route(d, x, w_router, bias, at<float>(ws, L.logits), ids, wts, offsets, sorted, pos, ws,
                    at<f16>(ws, L.x16), s));
  // the down GEMM writes each record's row times its routing weight in fp16
  f16* rows16 = at<f16>(ws, L.rows);
  TRY(enqueue_ffn(d, offsets, sorted, w, rows, ws, s, 0, rows16, wts));
  LAUNCH(MOE_KERNEL_COMBINE, s, moe::launch_combine16(rows16, pos, d.T, d.H, d.k, static_cast<uint16_t*>(y), s),
         "combine");
  return MOE_OK;
}

// Bytes of workspace moe_layer itself touches: every region up to the rows,
// whose fp16 half (the weighted fp16 rows) is all it uses.
size_t layout_rows16_bytes(const moe_dims& d) {
  return layout(d).rows + align256((size_t)d.T * d.k * d.H * 2);
}

// ---- moe_layer_noalloc: the workspace in a file-scope device array ------------
// For callers that cannot allocate device memory.  Every device that the
// library runs on holds its own copy of `scratch` until the process ends;
// its device address is looked up once per device (with that device
// current) and kept.  Host code uses only that address: the array's name in
// host code is a host-side stand-in, not a device address.
constexpr size_t NOALLOC_BYTES = MOE_NOALLOC_SCRATCH_BYTES;
static __device__ __align__(256) unsigned char scratch[NOALLOC_BYTES];
std::mutex g_scratch_mu;
void* g_scratch_ptr[SIDE_MAX_DEVICES] = {};

moe_status scratch_of_current_device(hipStream_t s, void** out) {
  int dev = -1;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return hip_fail(e, "hipGetDevice");
  if (dev < 0 || dev >= SIDE_MAX_DEVICES) return fail(MOE_ERR_ARG, "device %d is beyond the library's table", dev);
  if (s) {  // the kernels run on the stream's device: it must be the current one
    hipDevice_t sdev = -1;
    e = hipStreamGetDevice(s, &sdev);
    if (e != hipSuccess) return hip_fail(e, "hipStreamGetDevice");
    if ((int)sdev != dev) return fail(MOE_ERR_ARG, "stream is on device %d, the current device is %d", (int)sdev, dev);
  }
  std::lock_guard<std::mutex> lk(g_scratch_mu);
  if (!g_scratch_ptr[dev]) {
    void* p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess || !p) return hip_fail(e != hipSuccess ? e : hipErrorInvalidSymbol, "scratch address");
    g_scratch_ptr[dev] = p;
  }
  *out = g_scratch_ptr[dev];
  return MOE_OK;
}

}  // namespace

extern "C" {

moe_status moe_layer(moe_dims d, const void* x, const void* w_router, const float* bias, const moe_experts* w,
                     void* y, int32_t* topk_ids_out, float* topk_w_out, void* ws, size_t ws_bytes, void* stream) {
  TRY(check_dims(d));
  if (d.T == 0) return MOE_OK;
  TRY(check_layer_args(d, x, w_router, bias, w, y, topk_ids_out, topk_w_out));
  TRY(check_ws(d, ws, ws_bytes));
  return enqueue_layer(d, x, w_router, bias, w, y, topk_ids_out, topk_w_out, ws, (hipStream_t)stream);
}

moe_status moe_layer_noalloc(moe_dims d, const void* x, const void* w_router, const float* bias, const moe_experts* w,
                             void* y, int32_t* topk_ids_out, float* topk_w_out, void* stream) {
  TRY(check_dims(d));
  if (d.T == 0) return MOE_OK;
  TRY(check_layer_args(d, x, w_router, bias, w, y, topk_ids_out, topk_w_out));
  const size_t need = layout_rows16_bytes(d);
  if (need > NOALLOC_BYTES)
    return fail(MOE_ERR_WORKSPACE, "T = %d needs %zu bytes of scratch; the library's scratch holds %zu", d.T, need,
                NOALLOC_BYTES);
  hipStream_t s = (hipStream_t)stream;
  void* ws = nullptr;
  TRY(scratch_of_current_device(s, &ws));
  return enqueue_layer(d, x, w_router, bias, w, y, topk_ids_out, topk_w_out, ws, s);
}

size_t moe_layer_shared_workspace_bytes(moe_dims d, const moe_shared* shared) {
  if (check_dims(d) != MOE_OK || check_shared(shared) != MOE_OK) return 0;
  return shared_layout(d, *shared).total;
}

moe_status moe_layer_shared(moe_dims d, const moe_shared* shared, const void* x, const void* w_router,
                            const float* bias, const moe_experts* w, void* y, int32_t* topk_ids_out, float* topk_w_out,
                            void* ws, size_t ws_bytes, void* stream) {
  TRY(check_dims(d));
  TRY(check_shared(shared));
  if (d.T == 0) return MOE_OK;
  TRY(check_ptr(shared->w_gate_up, "shared w_gate_up"));
  TRY(check_ptr(shared->w_down, "shared w_down"));
  TRY(check_ptr(x, "x"));
  TRY(check_ptr(w_router, "w_router"));
  TRY(check_ptr(bias, "bias", false));
  TRY(check_experts(w));
  TRY(check_ptr(y, "y"));
  TRY(check_ptr(topk_ids_out, "topk_ids_out", false));
  TRY(check_ptr(topk_w_out, "topk_w_out", false));
  const SharedLayout SL = shared_layout(d, *shared);
  if (!ws) return fail(MOE_ERR_ARG, "workspace is NULL");
  if (!aligned16(ws)) return fail(MOE_ERR_ALIGN, "workspace is not 16-byte aligned");
  if (ws_bytes < SL.total) return fail(MOE_ERR_WORKSPACE, "workspace has %zu bytes, needs %zu", ws_bytes, SL.total);
  const Layout& L = SL.base;
  hipStream_t s = (hipStream_t)stream;
  const int T = d.T, H = d.H, width = shared->count * shared->I;
  int32_t* ids = topk_ids_out ? topk_ids_out : at<int32_t>(ws, L.ids);
  float* wts = topk_w_out ? topk_w_out : at<float>(ws, L.w);
  int32_t* offsets = at<int32_t>(ws, L.offsets);
  int32_t* sorted = at<int32_t>(ws, L.sorted);
  int32_t* pos = at<int32_t>(ws, L.pos);
  float* rows = at<float>(ws, L.rows);
  uint16_t* h = at<uint16_t>(ws, SL.h);
  float* dpart = at<float>(ws, SL.dpart);
  // the shared experts on every token (hidden layer, then the down partials),
  // on the side stream beside the routing and the routed experts.  From
  // SHARED_AFTER_ROUTE_T tokens the branch forks after the routing: both
  // branches are then compute-bound, and the shared GEMMs, started first,
  // held every CU while the latency-bound routing kernels waited for one.
  const bool route_first = T >= SHARED_AFTER_ROUTE_T;
  if (route_first)
    TRY(enqueue_route(d, x, w_router, bias, at<float>(ws, L.logits), ids, wts, offsets, sorted, pos, ws,
                      at<f16>(ws, L.x16), s));
  SideBranch branch(s);
  const hipStream_t s2 = branch.stream();
  LAUNCH(MOE_KERNEL_SHARED, s2,
         moe::launch_shared_hidden(static_cast<const uint16_t*>(x), static_cast<const uint16_t*>(shared->w_gate_up),
                                   at<float>(ws, SL.gupart), T, H, shared->count, shared->I,
                                   moe::router_plan(T, H, 2 * width), h, s2),
         "shared experts, gate/up");
  LAUNCH(MOE_KERNEL_SHARED, s2,
         moe::launch_router(h, static_cast<const uint16_t*>(shared->w_down), dpart, T, width, H,
                            moe::router_plan(T, width, H), s2),
         "shared experts, down");
  if (!route_first)
    TRY(enqueue_route(d, x, w_router, bias, at<float>(ws, L.logits), ids, wts, offsets, sorted, pos, ws,
                      at<f16>(ws, L.x16), s));
  f16* rows16 = at<f16>(ws, L.rows);
  TRY(enqueue_ffn(d, offsets, sorted, w, rows, ws, s, 0, rows16, wts));
  if (hipError_t e = branch.join(); e != hipSuccess) return hip_fail(e, "join of the shared experts");
  LAUNCH(MOE_KERNEL_COMBINE, s,
         moe::launch_combine16(rows16, pos, T, H, d.k, static_cast<uint16_t*>(y), s, dpart, SL.d_slabs), "combine");
  return MOE_OK;
}

size_t moe_latent_workspace_bytes(moe_dims d, int32_t H_model) {
  if (check_dims(d) != MOE_OK || check_latent_width(H_model) != MOE_OK) return 0;
  return latent_layout(d, H_model).total;
}

moe_status moe_latent_layer(moe_dims d, const moe_latent* lat, const void* x, const void* w_router, const float* bias,
                            const moe_experts* w, void* y, void* z_out, int32_t* topk_ids_out, float* topk_w_out,
                            void* ws, size_t ws_bytes, void* stream) {
  TRY(check_dims(d));
  if (!lat) return fail(MOE_ERR_ARG, "lat is NULL");
  TRY(check_latent_width(lat->H_model));
  if (d.T == 0) return MOE_OK;
  TRY(check_ptr(lat->w_down, "w_down"));
  TRY(check_ptr(lat->w_up, "w_up"));
  TRY(check_ptr(x, "x"));
  TRY(check_ptr(w_router, "w_router"));
  TRY(check_ptr(bias, "bias", false));
  TRY(check_experts(w));
  TRY(check_ptr(y, "y"));
  TRY(check_ptr(z_out, "z_out", false));
  TRY(check_ptr(topk_ids_out, "topk_ids_out", false));
  TRY(check_ptr(topk_w_out, "topk_w_out", false));
  const LatentLayout LL = latent_layout(d, lat->H_model);
  if (!ws) return fail(MOE_ERR_ARG, "workspace is NULL");
  if (!aligned16(ws)) return fail(MOE_ERR_ALIGN, "workspace is not 16-byte aligned");
  if (ws_bytes < LL.total) return fail(MOE_ERR_WORKSPACE, "workspace has %zu bytes, needs %zu", ws_bytes, LL.total);
  const Layout& L = LL.base;
  hipStream_t s = (hipStream_t)stream;
  const int T = d.T, H = d.H, Hm = lat->H_model, E = d.E, k = d.k;
  int32_t* ids = topk_ids_out ? topk_ids_out : at<int32_t>(ws, L.ids);
  float* wts = topk_w_out ? topk_w_out : at<float>(ws, L.w);
  int32_t* offsets = at<int32_t>(ws, L.offsets);
  int32_t* sorted = at<int32_t>(ws, L.sorted);
  int32_t* pos = at<int32_t>(ws, L.pos);
  f16* x16 = at<f16>(ws, L.x16);
  uint16_t* z = z_out ? static_cast<uint16_t*>(z_out) : at<uint16_t>(ws, LL.z);
  uint16_t* ylat = at<uint16_t>(ws, LL.ylat);
  float* rpart = at<float>(ws, LL.rpart);
  float* ppart = at<float>(ws, LL.ppart);
  // router on the hidden state
  const moe::RouterPlan rp = moe::router_plan(T, Hm, E);
  LAUNCH(MOE_KERNEL_ROUTER, s,
         moe::launch_router(static_cast<const uint16_t*>(x), static_cast<const uint16_t*>(w_router), rpart, T, Hm, E,
                            rp, s),
         "router");
  // routed-down projection: the latent in bf16 and its fp16 copy for the
  // experts.  (Beside the routing on the side stream it was slower: the
  // experts need it at once, so the join's latency is on the critical path.)
  LAUNCH(MOE_KERNEL_PROJECT, s,
         moe::launch_projection(static_cast<const uint16_t*>(x), static_cast<const uint16_t*>(lat->w_down), ppart, T,
                                Hm, H, moe::router_plan(T, Hm, H), z, x16, s),
         "routed-down projection");
  // top-k and permutation on the router's partials (x16 is already in place)
  if (moe::route_fused(T)) {
    LAUNCH(MOE_KERNEL_TOPK, s,
           moe::launch_route_small(rpart, rp.slabs, bias, at<float>(ws, L.logits), T, E, k, ids, wts, offsets, sorted,
                                   pos, at<int32_t>(ws, L.active), at<int32_t>(ws, L.nact), s),
           "route");
  } else {
    LAUNCH(MOE_KERNEL_TOPK, s,
           moe::launch_topk(rpart, rp.slabs, bias, at<float>(ws, L.logits), T, E, k, ids, wts, s), "top-k");
    LAUNCH(MOE_KERNEL_PERMUTE, s,
           moe::launch_permute(ids, T, E, k, at<uint64_t>(ws, L.masks), at<int32_t>(ws, L.counts),
                               at<int32_t>(ws, L.base), offsets, sorted, pos, at<int32_t>(ws, L.active),
                               at<int32_t>(ws, L.nact), at<int32_t>(ws, L.mtiles), at<int32_t>(ws, L.nmt), s),
           "permute");
  }
  float* rows = at<float>(ws, L.rows);
  f16* rows16 = at<f16>(ws, L.rows);
  TRY(enqueue_ffn(d, offsets, sorted, w, rows, ws, s, 0, rows16, wts));
  LAUNCH(MOE_KERNEL_COMBINE, s, moe::launch_combine16(rows16, pos, T, H, k, ylat, s), "combine");
  // routed-up projection back to the hidden width
  LAUNCH(MOE_KERNEL_PROJECT, s,
         moe::launch_projection(ylat, static_cast<const uint16_t*>(lat->w_up), ppart, T, H, Hm,
                                moe::router_plan(T, H, Hm), static_cast<uint16_t*>(y), nullptr, s),
         "routed-up projection");
  return MOE_OK;
}

moe_status moe_stream_read(const void* buf, size_t bytes, uint32_t* sink, void* stream) {
  if (!buf || !sink) return fail(MOE_ERR_ARG, "buf and sink must not be NULL");
  if (bytes == 0 || bytes % 16) return fail(MOE_ERR_ARG, "bytes = %zu must be a positive multiple of 16", bytes);
  if (!aligned16(buf)) return fail(MOE_ERR_ALIGN, "buf is not 16-byte aligned");
  if ((uintptr_t)sink & 3u) return fail(MOE_ERR_ALIGN, "sink is not 4-byte aligned");
  hipError_t e = moe::launch_stream_read(buf, (long long)bytes, sink, (hipStream_t)stream);
  if (e != hipSuccess) return hip_fail(e, "stream read");
  return MOE_OK;
}

moe_status moe_mfma_rate(int iters, float* sink, void* stream) {
  if (!sink) return fail(MOE_ERR_ARG, "sink must not be NULL");
  if (iters < 1 || iters > 10000000) return fail(MOE_ERR_ARG, "iters = %d must be in [1, 10^7]", iters);
  if ((uintptr_t)sink & 3u) return fail(MOE_ERR_ALIGN, "sink is not 4-byte aligned");
  hipError_t e = moe::launch_mfma_rate(iters, sink, (hipStream_t)stream);
  if (e != hipSuccess) return hip_fail(e, "mfma rate");
  return MOE_OK;
}

const char* moe_status_string(moe_status s) {
  switch (s) {
    case MOE_OK: return "ok";
    case MOE_ERR_ARG: return "invalid argument";
    case MOE_ERR_SHAPE: return "unsupported shape";
    case MOE_ERR_ALIGN: return "misaligned pointer";
    case MOE_ERR_WORKSPACE: return "workspace too small";
    case MOE_ERR_HIP: return "HIP error";
  }
  return "unknown status";
}

const char* moe_last_error(void) { return g_err; }

moe_status moe_profile_arm(moe_kernel kernel, int n_pairs) {
  g_prof.release();
  if ((int)kernel < 0 || (int)kernel >= MOE_KERNEL_COUNT || n_pairs < 1 || n_pairs > 65536)
    return fail(MOE_ERR_ARG, "moe_profile_arm: kernel %d, n_pairs %d", (int)kernel, n_pairs);
  g_prof.events.resize(2 * (size_t)n_pairs);
  for (size_t i = 0; i < g_prof.events.size(); i++) {
    if (hipEventCreateWithFlags(&g_prof.events[i], hipEventDisableSystemFence) != hipSuccess) {
      g_prof.events.resize(i);
      g_prof.release();
      return fail(MOE_ERR_HIP, "moe_profile_arm: hipEventCreateWithFlags failed");
    }
  }
  g_prof.kernel = (int)kernel;
  return MOE_OK;
}

int moe_profile_read(float* ms, int max) {
  if (!ms || max < 0) return -(int)fail(MOE_ERR_ARG, "moe_profile_read: ms is NULL or max < 0");
  const int n = g_prof.used < max ? g_prof.used : max;
  int status = n;
  for (int i = 0; i < n; i++) {
    if (hipEventSynchronize(g_prof.events[2 * i + 1]) != hipSuccess ||
        hipEventElapsedTime(&ms[i], g_prof.events[2 * i], g_prof.events[2 * i + 1]) != hipSuccess) {
      status = -(int)fail(MOE_ERR_HIP, "moe_profile_read: event %d", i);
      break;
    }
  }
  g_prof.release();
  return status;
}

}  // extern "C"
