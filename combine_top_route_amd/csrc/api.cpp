// C ABI of the fused MoE layer (declared in include/moe.h): host-side
// argument validation, workspace layout, launch sequencing, kernel timing.
//
// Every check runs before the first HIP call of an entry point, so a bad
// argument enqueues nothing.  The library owns no device memory: all buffers
// come from the caller, and the workspace is carved into fixed regions.
#include <algorithm>
#include <cstdarg>
#include <cstdio>
#include <cstring>
#include <limits>
#include <mutex>
#include <string>
#include <vector>

#include "common.h"
#include "moe.h"

using namespace moe;

namespace {

thread_local std::string g_err;

moe_status fail(moe_status s, const char* fmt, ...) {
  char buf[512];
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(buf, sizeof(buf), fmt, ap);
  va_end(ap);
  g_err = buf;
  return s;
}

moe_status hip_fail(hipError_t e, const char* where) {
  return fail(MOE_ERR_HIP, "%s: %s", where, hipGetErrorString(e));
}

// ------------------------------------------------------------------ timing
struct Rec {
  std::string name;
  hipEvent_t a, b;
};
std::mutex g_mu;
bool g_prof = false;
std::vector<Rec> g_recs;
std::vector<hipEvent_t> g_pool;

hipEvent_t pooled_event() {
  if (!g_pool.empty()) {
    hipEvent_t e = g_pool.back();
    g_pool.pop_back();
    return e;
  }
  hipEvent_t e = nullptr;
  if (hipEventCreate(&e) != hipSuccess) return nullptr;
  return e;
}

// Start and stop events for one kernel dispatch (see MOE_LAUNCH); a kernel
// whose events could not be created runs untimed and counts with 0 ms.
void prof_events(const char* name, hipEvent_t* start, hipEvent_t* stop) {
  std::lock_guard<std::mutex> lk(g_mu);
  Rec r;
  r.name = name;
  r.a = pooled_event();
  r.b = r.a ? pooled_event() : nullptr;
  if (!r.b) {
    if (r.a) g_pool.push_back(r.a);
    r.a = nullptr;
  }
  *start = r.a;
  *stop = r.b;
  g_recs.push_back(r);
}

LaunchCtx make_ctx(void* stream) {
  LaunchCtx c;
  c.stream = (hipStream_t)stream;
  bool prof;
  {
    std::lock_guard<std::mutex> lk(g_mu);
    prof = g_prof;
  }
  c.events = prof ? prof_events : nullptr;
  return c;
}

// ------------------------------------------------------------------ checks
constexpr int64_t kMaxT = int64_t(1) << 24;
constexpr int64_t kMaxR = int64_t(1) << 27;

moe_status check_shape(const moe_shape* s) {
  if (!s) return fail(MOE_ERR_INVALID_ARGUMENT, "shape is NULL");
  if (s->T < 1 || s->T > kMaxT) return fail(MOE_ERR_INVALID_ARGUMENT, "T=%lld outside [1, 2^24]", (long long)s->T);
  if (s->E < 1 || s->E > kMaxExperts)
    return fail(MOE_ERR_INVALID_ARGUMENT, "E=%lld outside [1, %d]", (long long)s->E, kMaxExperts);
  if (s->k < 1 || s->k > s->E) return fail(MOE_ERR_INVALID_ARGUMENT, "k=%lld outside [1, E=%lld]", (long long)s->k, (long long)s->E);
  if (s->T * s->k > kMaxR) return fail(MOE_ERR_INVALID_ARGUMENT, "T*k=%lld above 2^27", (long long)(s->T * s->k));
  if (s->d < 8 || s->d > 16384 || s->d % 8) return fail(MOE_ERR_INVALID_ARGUMENT, "d=%lld must be a multiple of 8 in [8, 16384]", (long long)s->d);
  if (s->I < 8 || s->I > 16384 || s->I % 8) return fail(MOE_ERR_INVALID_ARGUMENT, "I=%lld must be a multiple of 8 in [8, 16384]", (long long)s->I);
  if (s->dtype != MOE_F32 && s->dtype != MOE_BF16) return fail(MOE_ERR_INVALID_ARGUMENT, "dtype=%d unknown", s->dtype);
  if (s->logits_dtype != MOE_F32 && s->logits_dtype != MOE_BF16) return fail(MOE_ERR_INVALID_ARGUMENT, "logits_dtype=%d unknown", s->logits_dtype);
  if (s->precision < MOE_PREC_NATIVE || s->precision > MOE_PREC_FP8_BWD)
    return fail(MOE_ERR_INVALID_ARGUMENT, "precision=%d unknown", s->precision);
  if (s->flags & ~MOE_FLAG_PERSISTENT) return fail(MOE_ERR_INVALID_ARGUMENT, "flags=%d has unknown bits", (int)s->flags);
  if (!(s->swiglu_limit >= 0.0f && s->swiglu_limit <= std::numeric_limits<float>::max()))
    return fail(MOE_ERR_INVALID_ARGUMENT, "swiglu_limit=%g must be 0 (plain SwiGLU) or a positive finite clamp",
                (double)s->swiglu_limit);
  if (s->precision != MOE_PREC_NATIVE) {
    if (s->dtype != MOE_BF16) return fail(MOE_ERR_UNSUPPORTED, "fp8 precisions need dtype bf16");
    if (s->d % 128 || s->I % 128) return fail(MOE_ERR_UNSUPPORTED, "fp8 precisions need d and I multiples of 128");
    const int64_t widest = s->d > 2 * s->I ? s->d : 2 * s->I;
    if (s->T * s->k * (widest / 128) >= (int64_t(1) << 31))
      return fail(MOE_ERR_UNSUPPORTED, "fp8 precisions: T*k*max(d,2I)/128 must stay below 2^31");
  }
  return MOE_OK;
}

#define CHECK_PTR(p) \
  if (!(p)) return fail(MOE_ERR_INVALID_ARGUMENT, "%s is NULL", #p)

size_t elem_size(int dtype) { return dtype == MOE_F32 ? 4 : 2; }
// fp8 GEMMs in the forward / in the backward
bool fwd_fp8(const moe_shape* s) { return s->precision == MOE_PREC_FP8_BLOCK || s->precision == MOE_PREC_MXFP8; }
bool bwd_fp8(const moe_shape* s) { return s->precision != MOE_PREC_NATIVE; }
bool is_mx(const moe_shape* s) { return s->precision == MOE_PREC_MXFP8; }
// Scale bytes of an expert weight [N, K] encoded along K: blockwise fp32
// per 128 x 128 block, MX one byte per row and 32 columns.
size_t wscale_bytes(const moe_shape* s, int64_t N, int64_t K) {
  return is_mx(s) ? (size_t)(s->E * N * (K / 32)) : sizeof(float) * s->E * (N / 128) * (K / 128);
}
int dw_blocks(const moe_shape* s) {
  if (s->dtype == MOE_F32) return f32_dw_blocks((int)s->I);
  return bwd_fp8(s) ? fp8_dw_blocks((int)s->I) : bf16_dw_blocks((int)s->I);
}
// upper bound of the 128-row token blocks over all experts
int64_t nblk_max(const moe_shape* s) { return cdiv(s->T * s->k, kTokBlock) + s->E; }
size_t align256(size_t b) { return (b + 255) & ~size_t(255); }

// `saved`: H [R,2I] then Aw [R,I] (dtype); for fp8 also the weight codes and
// scales the backward's data gradients read: blockwise the forward encodings
// ([E,2I,d], [E,d,I]), MX the transposed ones ([E,d,2I], [E,I,d]).
struct SavedLayout {
  size_t H = 0, A = 0, wgu_dgq = 0, wd_dgq = 0, wgu_dgs = 0, wd_dgs = 0, total = 0;
};

SavedLayout saved_layout(const moe_shape* s) {
  SavedLayout L;
  const int64_t R = s->T * s->k, d = s->d, I = s->I, E = s->E;
  const size_t es = elem_size(s->dtype);
  L.H = 0;
  L.A = es * R * 2 * I;
  size_t off = L.A + es * R * I;
  if (fwd_fp8(s)) {
    auto take = [&](size_t bytes) {
      off = align256(off);
      const size_t o = off;
      off += bytes;
      return o;
    };
    L.wgu_dgq = take(E * d * 2 * I);
    L.wd_dgq = take(E * I * d);
    L.wgu_dgs = take(wscale_bytes(s, d, 2 * I));
    L.wd_dgs = take(wscale_bytes(s, I, d));
  }
  L.total = off;
  return L;
}

struct Layout {
  size_t hist = 0, tile_off = 0, order = 0, blk_off = 0, tiles = 0, tok = 0;  // routing / schedule
  size_t Y = 0, A = 0, H = 0;                             // forward
  size_t dH = 0, dXp = 0, dwp = 0, G = 0;                 // backward
  // fp8: quantised operands (q) and their scales (s)
  size_t xq = 0, xs = 0, wguq = 0, wgus = 0, wdq = 0, wds = 0, awq = 0, aws = 0;
  size_t doutq = 0, douts = 0, dhq = 0, dhs = 0;
  size_t tqa = 0, tsa = 0, tqb = 0, tsb = 0, Gf = 0;
  size_t wgu_dgq = 0, wgu_dgs = 0, wd_dgq = 0, wd_dgs = 0;  // fp8_bwd: the data gradients' weight codes
  size_t rsaved = 0;                                // recompute: the saved buffer
  size_t total = 0;
};

Layout layout(const moe_shape* s, int op) {
  Layout L;
  size_t off = 0;
  auto take = [&](size_t bytes) {
    size_t o = off;
    off += align256(bytes);
    return o;
  };
  const int64_t R = s->T * s->k;
  const size_t es = elem_size(s->dtype);
  const int64_t nchunks = cdiv(R, kSortChunk);
  L.tile_off = take(sizeof(int32_t) * (s->E + 1));
  L.order = take(sizeof(int32_t) * (s->E + 8 * cdiv(s->E, 8)));  // order, then xorder
  L.blk_off = take(sizeof(int32_t) * (s->E + 1));
  L.tiles = take(sizeof(int4) * max_row_tiles(R, s->E));
  if (op == MOE_OP_ROUTE || op == MOE_OP_FORWARD) L.hist = take(sizeof(int32_t) * nchunks * s->E);
  if (op == MOE_OP_FORWARD) {
    L.Y = take(es * R * s->d);
    L.A = take(es * R * s->I);
    if (s->dtype == MOE_F32) L.H = take(es * R * 2 * s->I);
  }
  const bool bwd = op == MOE_OP_BACKWARD || op == MOE_OP_BACKWARD_RECOMPUTE;
  if (bwd) {
    L.tok = take(sizeof(int32_t) * R);
    if (!bwd_fp8(s)) L.dH = take(es * R * 2 * s->I);  // the fp8 backward encodes dH in-kernel
    // the bf16 backward first writes the down GEMM's data gradient G [R, I]
    // into this buffer, which holds the permuted dx [R, d] only later
    const bool g_in_dxp = s->dtype == MOE_BF16 && !bwd_fp8(s);
    L.dXp = take(es * R * (g_in_dxp ? std::max(s->d, s->I) : s->d));
    L.dwp = take(sizeof(float) * R * dw_blocks(s));
    if (s->dtype == MOE_F32) L.G = take(sizeof(float) * R * s->I);
  }
  if (bwd_fp8(s)) {
    // row scales take one 32-bit word per 128 columns in both formats (an
    // fp32 scale, or four E8M0 bytes)
    const int64_t T = s->T, d = s->d, I = s->I, E = s->E;
    const size_t w = sizeof(uint32_t);
    // the recomputing backward reruns the gate/up GEMM with its x and weight codes
    if ((op == MOE_OP_FORWARD || op == MOE_OP_BACKWARD_RECOMPUTE) && fwd_fp8(s)) {
      L.xq = take(T * d);
      L.xs = take(w * R * (d / 128));  // per expert-sorted row
      L.wguq = take(E * 2 * I * d);
      L.wgus = take(wscale_bytes(s, 2 * I, d));
      if (op == MOE_OP_FORWARD) {
        L.wdq = take(E * d * I);
        L.wds = take(wscale_bytes(s, d, I));
        L.awq = take(R * I);
        L.aws = take(w * R * (I / 128));
      }
    }
    if (bwd) {
      const int64_t nb = nblk_max(s);
      L.doutq = take(T * d);
      L.douts = take(w * R * (d / 128));  // per expert-sorted row
      L.dhq = take(R * 2 * I);
      L.dhs = take(w * R * (2 * I / 128));
      const int64_t ra = d > 2 * I ? d : 2 * I, rb = d > I ? d : I;
      L.tqa = take(ra * nb * kTokBlock);
      L.tsa = take(w * ra * nb);
      L.tqb = take(rb * nb * kTokBlock);
      L.tsb = take(w * rb * nb);
      L.Gf = take(sizeof(float) * R * I);
      if (!fwd_fp8(s)) {
        L.wgu_dgq = take(E * d * 2 * I);
        L.wd_dgq = take(E * I * d);
        L.wgu_dgs = take(wscale_bytes(s, d, 2 * I));
        L.wd_dgs = take(wscale_bytes(s, I, d));
      }
    }
  }
  if (op == MOE_OP_BACKWARD_RECOMPUTE) L.rsaved = take(saved_layout(s).total);
  L.total = off;
  return L;
}

Fp8Saved fp8_saved(const moe_shape* s, const void* saved) {
  Fp8Saved v = {};
  if (!saved) return v;
  const SavedLayout L = saved_layout(s);
  char* b = (char*)saved;
  v.wgu_dgq = (uint8_t*)(b + L.wgu_dgq);
  v.wd_dgq = (uint8_t*)(b + L.wd_dgq);
  v.wgu_dgs = b + L.wgu_dgs;
  v.wd_dgs = b + L.wd_dgs;
  return v;
}

moe_status check_routing(const moe_routing* r, bool need_all) {
  CHECK_PTR(r);
  CHECK_PTR(r->topk_ids);
  CHECK_PTR(r->topk_w);
  CHECK_PTR(r->counts);
  CHECK_PTR(r->offsets);
  CHECK_PTR(r->row_of);
  CHECK_PTR(r->src_of);
  (void)need_all;
  return MOE_OK;
}

moe_status check_ws(const moe_shape* s, int op, void* ws, size_t bytes) {
  const size_t need = layout(s, op).total;
  if (bytes < need) return fail(MOE_ERR_WORKSPACE, "workspace of %zu bytes, %zu needed", bytes, need);
  if (need && !ws) return fail(MOE_ERR_INVALID_ARGUMENT, "workspace is NULL");
  if (((uintptr_t)ws) & 255) return fail(MOE_ERR_INVALID_ARGUMENT, "workspace must be 256-byte aligned");
  return MOE_OK;
}

moe_status check_aligned16(const void* p, const char* name) {
  if (((uintptr_t)p) & 15) return fail(MOE_ERR_INVALID_ARGUMENT, "%s must be 16-byte aligned", name);
  return MOE_OK;
}

#define TRY(x)                          \
  do {                                  \
    moe_status _s = (x);                \
    if (_s != MOE_OK) return _s;        \
  } while (0)

#define HIP_TRY(x, where)                      \
  do {                                         \
    hipError_t _e = (x);                       \
    if (_e != hipSuccess) return hip_fail(_e, where); \
  } while (0)

char* at(void* base, size_t off) { return (char*)base + off; }

// routing launches shared by moe_route, moe_route_noalloc and moe_forward;
// hist: the counting sort's per-chunk histograms [ceil(T*k/kSortChunk), E]
moe_status run_route(const moe_shape* s, moe_routing* r, int32_t* hist, const LaunchCtx& c) {
  const int T = (int)s->T, E = (int)s->E, k = (int)s->k;
  if (r->logits) HIP_TRY(launch_topk(c, r->logits, s->logits_dtype, T, E, k, r->topk_ids, r->topk_w), "route_topk");
  HIP_TRY(launch_sort(c, r->topk_ids, T, E, k, hist, r->counts, r->offsets, r->row_of, r->src_of),
          "route_sort");
  return MOE_OK;
}

// ------------------------------------------------------------ no-allocation routing
// moe_route_noalloc keeps the histograms in this file-scope device array
// instead of a caller workspace.  In host code `scratch` names a host-side
// stand-in, not device memory: its device address comes from
// hipGetSymbolAddress, taken once per device with that device current, and
// only that address is handed to kernels.
constexpr size_t kNoAllocScratchBytes = size_t(4) << 20;
static __device__ __align__(256) uint8_t scratch[kNoAllocScratchBytes];

constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void* g_scratch_ptr[kMaxDevices] = {};

// Device address of `scratch` on the current device (looked up on the
// first call per device).
moe_status scratch_on_current_device(void** ptr) {
  int dev = -1;
  HIP_TRY(hipGetDevice(&dev), "hipGetDevice");
  if (dev < 0 || dev >= kMaxDevices) return fail(MOE_ERR_UNSUPPORTED, "device %d beyond %d", dev, kMaxDevices);
  std::lock_guard<std::mutex> lk(g_scratch_mu);
  if (!g_scratch_ptr[dev]) {
    void* p = nullptr;
    HIP_TRY(hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)), "hipGetSymbolAddress(scratch)");
    if (!p) return fail(MOE_ERR_HIP, "hipGetSymbolAddress(scratch) gave a null address");
    g_scratch_ptr[dev] = p;
  }
  *ptr = g_scratch_ptr[dev];
  return MOE_OK;
}

LayerArgs layer_args(const moe_shape* s, const moe_routing* r, const void* x, const void* wgu,
                     const void* wd, void* ws, const Layout& L) {
  LayerArgs a;
  a.T = (int)s->T;
  a.d = (int)s->d;
  a.E = (int)s->E;
  a.k = (int)s->k;
  a.I = (int)s->I;
  a.R = (int)(s->T * s->k);
  a.dtype = s->dtype;
  a.x = x;
  a.w_gate_up = wgu;
  a.w_down = wd;
  a.topk_w = r->topk_w;
  a.offsets = r->offsets;
  a.src_of = r->src_of;
  a.row_of = r->row_of;
  a.tile_off = (const int32_t*)at(ws, L.tile_off);
  a.tiles = (const int4*)at(ws, L.tiles);
  a.order = (const int32_t*)at(ws, L.order);
  a.xorder = a.order + s->E;
  a.tok_of = L.tok ? (const int32_t*)at(ws, L.tok) : nullptr;  // backward layouts only
  a.swiglu_lim = s->swiglu_limit > 0.0f ? s->swiglu_limit : __builtin_huge_valf();
  a.persistent = (s->flags & MOE_FLAG_PERSISTENT) != 0;
  return a;
}

// The forward's GEMMs (and, fp8, its encodings) writing H (may be null for
// bf16), A and, unless Y is null, Y.  Y == null: the gate/up half alone,
// as the recomputing backward needs it.  saved: where the fp8 forward leaves
// the transposed weight codes (null: not kept).
hipError_t forward_gemms(const moe_shape* shape, const LaunchCtx& c, const LayerArgs& a, void* ws,
                         const Layout& L, void* saved, void* H, void* A, void* Y) {
  if (shape->dtype == MOE_F32) return f32_fwd_gemms(c, a, H, A, Y);
  if (!fwd_fp8(shape)) return bf16_fwd_gemms(c, a, H, A, Y);
  Fp8Fwd q;
  q.mx = is_mx(shape);
  q.xq = (uint8_t*)at(ws, L.xq); q.xs = at(ws, L.xs);
  q.wguq = (uint8_t*)at(ws, L.wguq); q.wgus = at(ws, L.wgus);
  q.wdq = Y ? (uint8_t*)at(ws, L.wdq) : nullptr; q.wds = Y ? at(ws, L.wds) : nullptr;
  q.awq = Y ? (uint8_t*)at(ws, L.awq) : nullptr; q.aws = Y ? at(ws, L.aws) : nullptr;
  q.sv = fp8_saved(shape, saved);
  return fp8_fwd_gemms(c, a, q, H, A, Y);
}

}  // namespace

extern "C" {

moe_status moe_workspace_size(const moe_shape* shape, int op, size_t* bytes) {
  TRY(check_shape(shape));
  CHECK_PTR(bytes);
  if (op < MOE_OP_ROUTE || op > MOE_OP_BACKWARD_RECOMPUTE) return fail(MOE_ERR_INVALID_ARGUMENT, "op=%d unknown", op);
  *bytes = layout(shape, op).total;
  return MOE_OK;
}

moe_status moe_saved_size(const moe_shape* shape, size_t* bytes) {
  TRY(check_shape(shape));
  CHECK_PTR(bytes);
  *bytes = saved_layout(shape).total;
  return MOE_OK;
}

size_t moe_workspace_bytes(const moe_shape* shape, int op) {
  size_t n = 0;
  return moe_workspace_size(shape, op, &n) == MOE_OK ? n : 0;
}

size_t moe_saved_bytes(const moe_shape* shape) {
  size_t n = 0;
  return moe_saved_size(shape, &n) == MOE_OK ? n : 0;
}

moe_status moe_route(const moe_shape* shape, moe_routing* routing, void* workspace,
                     size_t workspace_bytes, void* stream) {
  TRY(check_shape(shape));
  TRY(check_routing(routing, true));
  TRY(check_ws(shape, MOE_OP_ROUTE, workspace, workspace_bytes));
  const Layout L = layout(shape, MOE_OP_ROUTE);
  (void)hipGetLastError();
  return run_route(shape, routing, (int32_t*)at(workspace, L.hist), make_ctx(stream));
}

moe_status moe_route_noalloc(const moe_shape* shape, moe_routing* routing, void* stream) {
  TRY(check_shape(shape));
  TRY(check_routing(routing, true));
  const size_t need = sizeof(int32_t) * cdiv(shape->T * shape->k, kSortChunk) * shape->E;
  if (need > kNoAllocScratchBytes)
    return fail(MOE_ERR_UNSUPPORTED,
                "moe_route_noalloc: T*k=%lld, E=%lld need %zu bytes of scratch, above its %zu; "
                "use moe_route with a workspace", (long long)(shape->T * shape->k), (long long)shape->E,
                need, kNoAllocScratchBytes);
  void* hist = nullptr;
  TRY(scratch_on_current_device(&hist));
  (void)hipGetLastError();
  return run_route(shape, routing, (int32_t*)hist, make_ctx(stream));
}

moe_status moe_forward(const moe_shape* shape, const void* x, moe_routing* routing,
                       const void* w_gate_up, const void* w_down, void* out, void* saved,
                       void* workspace, size_t workspace_bytes, void* stream) {
  TRY(check_shape(shape));
  CHECK_PTR(x);
  CHECK_PTR(w_gate_up);
  CHECK_PTR(w_down);
  CHECK_PTR(out);
  TRY(check_routing(routing, true));
  TRY(check_ws(shape, MOE_OP_FORWARD, workspace, workspace_bytes));
  TRY(check_aligned16(x, "x"));
  TRY(check_aligned16(w_gate_up, "w_gate_up"));
  TRY(check_aligned16(w_down, "w_down"));
  TRY(check_aligned16(out, "out"));
  if (saved) TRY(check_aligned16(saved, "saved"));
  const Layout L = layout(shape, MOE_OP_FORWARD);
  const LaunchCtx c = make_ctx(stream);
  (void)hipGetLastError();
  TRY(run_route(shape, routing, (int32_t*)at(workspace, L.hist), c));
  HIP_TRY(launch_schedule(c, routing->offsets, (int)shape->E, (int32_t*)at(workspace, L.tile_off),
                          (int32_t*)at(workspace, L.order), nullptr, nullptr, (int4*)at(workspace, L.tiles)),
          "route_schedule");
  const LayerArgs a = layer_args(shape, routing, x, w_gate_up, w_down, workspace, L);
  const size_t es = elem_size(shape->dtype);
  const int64_t R = shape->T * shape->k;
  void* H = saved ? saved : (shape->dtype == MOE_F32 ? at(workspace, L.H) : nullptr);
  void* A = saved ? at(saved, es * R * 2 * shape->I) : at(workspace, L.A);
  void* Y = at(workspace, L.Y);
  HIP_TRY(forward_gemms(shape, c, a, workspace, L, saved, H, A, Y), "forward GEMMs");
  // rows already carry their top-k weight: the combine is a plain sum
  HIP_TRY(launch_combine(c, "combine", shape->dtype, Y, routing->row_of, nullptr, (int)shape->T,
                         (int)shape->k, (int)shape->d, out), "combine");
  return MOE_OK;
}

moe_status moe_backward(const moe_shape* shape, const void* dout, const void* x,
                        const moe_routing* routing, const void* w_gate_up, const void* w_down,
                        const void* saved, void* dx, void* dw_gate_up, void* dw_down,
                        float* d_topk_w, void* dlogits, void* workspace, size_t workspace_bytes,
                        void* stream) {
  TRY(check_shape(shape));
  CHECK_PTR(dout);
  CHECK_PTR(x);
  CHECK_PTR(w_gate_up);
  CHECK_PTR(w_down);
  CHECK_PTR(dx);
  CHECK_PTR(dw_gate_up);
  CHECK_PTR(dw_down);
  CHECK_PTR(d_topk_w);
  TRY(check_routing(routing, true));
  if (dlogits && !routing->logits)
    return fail(MOE_ERR_INVALID_ARGUMENT, "dlogits needs the logits form of routing");
  const int op = saved ? MOE_OP_BACKWARD : MOE_OP_BACKWARD_RECOMPUTE;
  TRY(check_ws(shape, op, workspace, workspace_bytes));
  TRY(check_aligned16(dout, "dout"));
  TRY(check_aligned16(x, "x"));
  TRY(check_aligned16(w_gate_up, "w_gate_up"));
  TRY(check_aligned16(w_down, "w_down"));
  if (saved) TRY(check_aligned16(saved, "saved"));
  TRY(check_aligned16(dx, "dx"));
  TRY(check_aligned16(dw_gate_up, "dw_gate_up"));
  TRY(check_aligned16(dw_down, "dw_down"));
  const Layout L = layout(shape, op);
  const LaunchCtx c = make_ctx(stream);
  (void)hipGetLastError();
  HIP_TRY(launch_schedule(c, routing->offsets, (int)shape->E, (int32_t*)at(workspace, L.tile_off),
                          (int32_t*)at(workspace, L.order), (int32_t*)at(workspace, L.order) + shape->E,
                          bwd_fp8(shape) ? (int32_t*)at(workspace, L.blk_off) : nullptr,
                          (int4*)at(workspace, L.tiles)),
          "route_schedule");
  HIP_TRY(launch_tok_of(c, routing->src_of, (int)(shape->T * shape->k), (int)shape->k,
                        (int32_t*)at(workspace, L.tok)), "route_tok");
  const LayerArgs a = layer_args(shape, routing, x, w_gate_up, w_down, workspace, L);
  const size_t es = elem_size(shape->dtype);
  const int64_t R = shape->T * shape->k;
  if (!saved) {  // recompute what the forward saves: H, Aw (and the fp8 weight codes)
    void* rs = at(workspace, L.rsaved);
    HIP_TRY(forward_gemms(shape, c, a, workspace, L, rs, rs, at(rs, es * R * 2 * shape->I), nullptr),
            "recompute GEMMs");
    saved = rs;
  }
  const void* H = saved;
  const void* A = (const char*)saved + es * R * 2 * shape->I;
  void* dH = at(workspace, L.dH);
  void* dXp = at(workspace, L.dXp);
  float* dwp = (float*)at(workspace, L.dwp);
  if (shape->dtype == MOE_F32)
    HIP_TRY(f32_bwd_gemms(c, a, dout, H, A, dH, dXp, dwp, dw_gate_up, dw_down,
                          (float*)at(workspace, L.G)), "backward GEMMs");
  else if (bwd_fp8(shape)) {
    Fp8Bwd q;
    q.mx = is_mx(shape);
    q.quant_weights = !fwd_fp8(shape);
    q.doutq = (uint8_t*)at(workspace, L.doutq); q.douts = at(workspace, L.douts);
    if (q.quant_weights) {
      q.sv.wgu_dgq = (uint8_t*)at(workspace, L.wgu_dgq); q.sv.wgu_dgs = at(workspace, L.wgu_dgs);
      q.sv.wd_dgq = (uint8_t*)at(workspace, L.wd_dgq); q.sv.wd_dgs = at(workspace, L.wd_dgs);
    } else {
      q.sv = fp8_saved(shape, saved);
    }
    q.dhq = (uint8_t*)at(workspace, L.dhq); q.dhs = at(workspace, L.dhs);
    q.tqa = (uint8_t*)at(workspace, L.tqa); q.tsa = at(workspace, L.tsa);
    q.tqb = (uint8_t*)at(workspace, L.tqb); q.tsb = at(workspace, L.tsb);
    q.G = (float*)at(workspace, L.Gf);
    q.blk_off = (const int32_t*)at(workspace, L.blk_off);
    q.nblk_max = (int)nblk_max(shape);
    HIP_TRY(fp8_bwd_gemms(c, a, q, dout, H, A, dXp, dwp, dw_gate_up, dw_down), "backward GEMMs");
  } else
    HIP_TRY(bf16_bwd_gemms(c, a, dout, H, A, dH, dXp, dwp, dw_gate_up, dw_down), "backward GEMMs");
  HIP_TRY(launch_topk_grad(c, dwp, dw_blocks(shape), routing->row_of, routing->topk_ids,
                           routing->topk_w, (int)shape->T, (int)shape->k, (int)shape->E, d_topk_w,
                           dlogits, shape->logits_dtype), "topk_grad");
  HIP_TRY(launch_combine(c, "reduce_dx", shape->dtype, dXp, routing->row_of, nullptr, (int)shape->T,
                         (int)shape->k, (int)shape->d, dx), "reduce_dx");
  return MOE_OK;
}

moe_status moe_permute(const moe_shape* shape, const void* x, const moe_routing* routing,
                       void* xp, void* stream) {
  TRY(check_shape(shape));
  CHECK_PTR(x);
  CHECK_PTR(xp);
  CHECK_PTR(routing);
  CHECK_PTR(routing->src_of);
  CHECK_PTR(routing->row_of);
  TRY(check_aligned16(x, "x"));
  TRY(check_aligned16(xp, "xp"));
  const LaunchCtx c = make_ctx(stream);
  (void)hipGetLastError();
  HIP_TRY(launch_permute(c, "permute", shape->dtype, x, routing->src_of, routing->row_of,
                         (int)(shape->T * shape->k), (int)shape->k, (int)shape->d, xp), "permute");
  return MOE_OK;
}

moe_status moe_combine(const moe_shape* shape, const void* rows, const moe_routing* routing,
                       void* out, void* stream) {
  TRY(check_shape(shape));
  CHECK_PTR(rows);
  CHECK_PTR(out);
  CHECK_PTR(routing);
  CHECK_PTR(routing->row_of);
  CHECK_PTR(routing->topk_w);
  TRY(check_aligned16(rows, "rows"));
  TRY(check_aligned16(out, "out"));
  const LaunchCtx c = make_ctx(stream);
  (void)hipGetLastError();
  HIP_TRY(launch_combine(c, "combine_weighted", shape->dtype, rows, routing->row_of, routing->topk_w, (int)shape->T,
                         (int)shape->k, (int)shape->d, out), "combine");
  return MOE_OK;
}

}  // extern "C"

namespace {

moe_status quantize_common(bool mx, int kind, const void* src, int64_t n0, int64_t n1, int64_t n2,
                           uint8_t* q, void* s, void* stream) {
  CHECK_PTR(src);
  CHECK_PTR(q);
  CHECK_PTR(s);
  if (kind != MOE_QUANT_ROWS && kind != MOE_QUANT_WEIGHT && kind != MOE_QUANT_WEIGHT_T)
    return fail(MOE_ERR_INVALID_ARGUMENT, "kind=%d unknown", kind);
  if (n0 < 1 || n1 < 1 || (kind != MOE_QUANT_ROWS && n2 < 1))
    return fail(MOE_ERR_INVALID_ARGUMENT, "extents must be positive");
  if (kind == MOE_QUANT_ROWS) {
    if (n1 % 128) return fail(MOE_ERR_INVALID_ARGUMENT, "n1=%lld must be a multiple of 128", (long long)n1);
    if (n0 > (int64_t(1) << 31) / (n1 / 128)) return fail(MOE_ERR_INVALID_ARGUMENT, "too many blocks");
  } else {
    if (n1 % 128 || n2 % 128)
      return fail(MOE_ERR_INVALID_ARGUMENT, "n1=%lld and n2=%lld must be multiples of 128", (long long)n1,
                  (long long)n2);
    if (n0 > 65535 || n1 > 65535 * 128 || n2 > 65535 * 128)
      return fail(MOE_ERR_INVALID_ARGUMENT, "weight extents too large");
  }
  TRY(check_aligned16(src, "src"));
  TRY(check_aligned16(q, "q"));
  if (((uintptr_t)s) & 3) return fail(MOE_ERR_INVALID_ARGUMENT, "s must be 4-byte aligned");
  const LaunchCtx c = make_ctx(stream);
  (void)hipGetLastError();
  if (kind == MOE_QUANT_ROWS) {
    HIP_TRY(launch_quant_rows(c, "quant_rows", src, n1, n0, (int)n1, q, s, mx, false), "quant_rows");
    return MOE_OK;
  }
  const bool tr = kind == MOE_QUANT_WEIGHT_T;
  uint8_t* fq = tr ? nullptr : q;
  uint8_t* tq = tr ? q : nullptr;
  void* fs = tr ? nullptr : s;
  void* ts = tr ? s : nullptr;
  if (mx)
    HIP_TRY(launch_quant_weight_mx(c, "quant_weight", src, (int)n0, (int)n1, (int)n2, fq, (uint8_t*)fs,
                                   tq, (uint8_t*)ts, false), "quant_weight");
  else
    HIP_TRY(launch_quant_weight(c, "quant_weight", src, (int)n0, (int)n1, (int)n2, fq, (float*)fs, tq,
                                (float*)ts), "quant_weight");
  return MOE_OK;
}

moe_status quantize_tokens_common(bool mx, const moe_shape* shape, const void* src, int64_t C,
                                  int gather, const moe_routing* routing, uint8_t* q, void* s,
                                  void* workspace, size_t workspace_bytes, void* stream) {
  TRY(check_shape(shape));
  CHECK_PTR(src);
  CHECK_PTR(q);
  CHECK_PTR(s);
  CHECK_PTR(routing);
  CHECK_PTR(routing->offsets);
  if (gather) CHECK_PTR(routing->src_of);
  if (shape->dtype != MOE_BF16) return fail(MOE_ERR_UNSUPPORTED, "token-block quantisation reads bf16");
  if (C < 128 || C > 65535 * 64 || C % 128)
    return fail(MOE_ERR_INVALID_ARGUMENT, "C=%lld must be a positive multiple of 128", (long long)C);
  TRY(check_ws(shape, MOE_OP_ROUTE, workspace, workspace_bytes));
  TRY(check_aligned16(src, "src"));
  TRY(check_aligned16(q, "q"));
  if (((uintptr_t)s) & 3) return fail(MOE_ERR_INVALID_ARGUMENT, "s must be 4-byte aligned");
  const Layout L = layout(shape, MOE_OP_ROUTE);
  const LaunchCtx c = make_ctx(stream);
  (void)hipGetLastError();
  int32_t* blk_off = (int32_t*)at(workspace, L.blk_off);
  HIP_TRY(launch_schedule(c, routing->offsets, (int)shape->E, (int32_t*)at(workspace, L.tile_off),
                          (int32_t*)at(workspace, L.order), nullptr, blk_off, nullptr), "route_schedule");
  HIP_TRY(launch_quant_tok(c, "quant_tokens", src, C, gather ? routing->src_of : nullptr,
                           (int)shape->k, (int)C, routing->offsets, blk_off, (int)shape->E,
                           (int)nblk_max(shape), q, s, mx, false), "quant_tokens");
  return MOE_OK;
}

}  // namespace

extern "C" {

moe_status moe_quantize_fp8(int kind, const void* src, int64_t n0, int64_t n1, int64_t n2,
                            uint8_t* q, float* s, void* stream) {
  return quantize_common(false, kind, src, n0, n1, n2, q, s, stream);
}

moe_status moe_quantize_mxfp8(int kind, const void* src, int64_t n0, int64_t n1, int64_t n2,
                              uint8_t* q, uint8_t* s, void* stream) {
  return quantize_common(true, kind, src, n0, n1, n2, q, s, stream);
}

moe_status moe_quantize_tokens_fp8(const moe_shape* shape, const void* src, int64_t C, int gather,
                                   const moe_routing* routing, uint8_t* q, float* s, void* workspace,
                                   size_t workspace_bytes, void* stream) {
  return quantize_tokens_common(false, shape, src, C, gather, routing, q, s, workspace,
                                workspace_bytes, stream);
}

moe_status moe_quantize_tokens_mxfp8(const moe_shape* shape, const void* src, int64_t C, int gather,
                                     const moe_routing* routing, uint8_t* q, uint8_t* s,
                                     void* workspace, size_t workspace_bytes, void* stream) {
  return quantize_tokens_common(true, shape, src, C, gather, routing, q, s, workspace,
                                workspace_bytes, stream);
}

const char* moe_status_string(moe_status s) {
  switch (s) {
    case MOE_OK: return "MOE_OK";
    case MOE_ERR_INVALID_ARGUMENT: return "MOE_ERR_INVALID_ARGUMENT";
    case MOE_ERR_UNSUPPORTED: return "MOE_ERR_UNSUPPORTED";
    case MOE_ERR_WORKSPACE: return "MOE_ERR_WORKSPACE";
    case MOE_ERR_HIP: return "MOE_ERR_HIP";
  }
  return "MOE_ERR_UNKNOWN";
}

const char* moe_last_error(void) { return g_err.c_str(); }

moe_status moe_profile_begin(void) {
  std::lock_guard<std::mutex> lk(g_mu);
  g_prof = true;
  for (auto& r : g_recs) {
    if (r.a) g_pool.push_back(r.a);
    if (r.b) g_pool.push_back(r.b);
  }
  g_recs.clear();
  return MOE_OK;
}

moe_status moe_profile_end(moe_kernel_stat* stats, int capacity, int* count) {
  std::lock_guard<std::mutex> lk(g_mu);
  g_prof = false;
  std::vector<moe_kernel_stat> agg;
  for (auto& r : g_recs) {
    float ms = 0.0f;
    if (r.a && r.b) {
      hipError_t e = hipEventSynchronize(r.b);
      if (e == hipSuccess) e = hipEventElapsedTime(&ms, r.a, r.b);
      if (e != hipSuccess) return hip_fail(e, "profile events");
    }
    size_t i = 0;
    for (; i < agg.size(); ++i)
      if (r.name == agg[i].name) break;
    if (i == agg.size()) {
      moe_kernel_stat s;
      std::memset(&s, 0, sizeof(s));
      std::strncpy(s.name, r.name.c_str(), sizeof(s.name) - 1);
      agg.push_back(s);
    }
    agg[i].launches += 1;
    agg[i].total_ms += ms;
    if (r.a) g_pool.push_back(r.a);
    if (r.b) g_pool.push_back(r.b);
  }
  g_recs.clear();
  for (int i = 0; i < (int)agg.size() && i < capacity; ++i) stats[i] = agg[i];
  if (count) *count = (int)agg.size();
  return MOE_OK;
}

}  // extern "C"
