// C ABI of the MoE layer library (declarations and contract: include/moe.h).
// Validation, workspace layout and stream-ordered launches; no allocation and
// no host synchronisation on the forward path.
#include <hip/hip_runtime.h>
#include <stdarg.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

#include <string>
#include <vector>

#include "moe_internal.h"

using namespace qreb;

struct moe_ctx {
  moe_config cfg;
  LayerDev d;
  bool has_weights = false;
  std::string err;
  // kernel timing: events [call][slot][begin/end]
  std::vector<hipEvent_t> ev;
  std::vector<uint8_t> launched;  // [call][slot]
  int prof_max = 0, prof_calls = 0;
  uint32_t prof_mask = 0xffu;   // slots that get event pairs
  // matrix-core work runs on this stream, forked from and joined back into the
  // caller's stream with two events (created at open, default priority)
  hipStream_t side = nullptr;
  hipEvent_t fork = nullptr, join = nullptr;
  // this device's copy of the library's static scratch (moe_forward_noalloc)
  uint8_t* scratch = nullptr;
  // expert cache: the stream that prefetches into this context's slots (a
  // lookahead from the previous layer), and the event its next forward waits on
  hipStream_t copy = nullptr;
  hipEvent_t pf_done = nullptr;
  bool pf_pending = false;
  uint32_t cache_flags = 0;
};

// The device-side address of a buffer the kernels may read: device memory as
// it is; host memory only if it is pinned and mapped (its device alias).
static const void* device_view(const void* p) {
  hipPointerAttribute_t a;
  if (hipPointerGetAttributes(&a, p) != hipSuccess) {
    (void)hipGetLastError();
    return nullptr;
  }
  if (a.type == hipMemoryTypeDevice || a.type == hipMemoryTypeManaged) return p;
  if (a.type == hipMemoryTypeHost) {
    void* dp = nullptr;
    if (hipHostGetDevicePointer(&dp, const_cast<void*>(p), 0) != hipSuccess) {
      (void)hipGetLastError();
      return nullptr;
    }
    return dp;
  }
  return nullptr;
}

static void prof_clear(moe_ctx* c) {
  for (hipEvent_t e : c->ev) (void)hipEventDestroy(e);
  c->ev.clear();
  c->launched.clear();
  c->prof_max = c->prof_calls = 0;
}

namespace qreb {

int router_ksplit(int hidden) { return (hidden / kGroup + kRouterGPW - 1) / kRouterGPW; }

// Tokens per router GEMV workgroup: at most kRouterTokMax, and at most
// 4096 / Epad (the top-k pass holds a token block's logits in LDS).
int router_tok_block(int n_tokens, int e_pad) {
  int tb = 4096 / e_pad;
  if (tb > kRouterTokMax) tb = kRouterTokMax;
  // decode-sized batches: one token per workgroup up to 16 tokens, four up
  // to 64, for more workgroups on the router weights (each re-reads them
  // from cache); one token measured 1.5 us faster than four at 4 and 16
  if (n_tokens <= 16) tb = 1;
  else if (n_tokens <= 64 && tb > 4) tb = 4;
  if (tb < 1) tb = 1;
  return n_tokens < tb ? n_tokens : tb;
}

static size_t al(size_t v) { return (v + 255) & ~size_t(255); }

WsLayout ws_layout(const moe_config& c) {
  WsLayout L{};
  const size_t T = (size_t)c.max_tokens, H = (size_t)c.hidden, E = (size_t)c.n_experts;
  const size_t k = (size_t)c.top_k, I = (size_t)c.inter;
  const size_t Is = (c.flags & MOE_F_SHARED) ? (size_t)c.shared_inter : 0;
  const size_t Epad = (E + 63) / 64 * 64, G = H / 64;
  const size_t KS = (size_t)router_ksplit(c.hidden);
  const size_t Tk = T * k, Ts = (c.flags & MOE_F_SHARED) ? T : 0;
  size_t o = 0;
  auto take = [&](size_t bytes) {
    size_t r = o;
    o += al(bytes);
    return r;
  };
  L.part = take(KS * T * Epad * 4);
  L.x16 = take(T * H * 2);
  L.xs = take(T * G * 8);
  L.ids = take(Tk * 4);
  L.p = take(Tk * 4);
  L.misc = take(kMiscInts * 4);   // zeroed at bind time
  L.offs = take((E + 1) * 4);
  L.slots = take((Tk + T) * 4);
  L.items = take((E + 1) * 32);   // (expert, rows, offset, 0) + first 4 slots
  L.mitems = take((E + 1) * 16);
  {   // wide unit lists, one per XCD: routed tiles (rt bounds them) and shared tiles
    const int rt = (int)((Tk + kMfmaBM - 1) / kMfmaBM + E + 1), st = Ts ? (int)((T + kMfmaBM - 1) / kMfmaBM) : 0;
    L.cap_up = wide_cap(rt + st, st, (int)((I + kWideColsUp - 1) / kWideColsUp),
                        (int)((Is + kWideColsUp - 1) / kWideColsUp));
    L.cap_dn = wide_cap(rt + st, 0, (int)((H + kWideColsDn - 1) / kWideColsDn), 0);
    L.wunits_up = take((size_t)8 * L.cap_up * 16);
    L.wunits_dn = take((size_t)8 * L.cap_dn * 16);
  }
  L.ntiles = take(((Tk + kNarrowBM - 1) / kNarrowBM + E + (T + kNarrowBM - 1) / kNarrowBM + 1) * 8);
  L.pred = take(Tk * 4);
  L.hbuf = take((Tk * I + Ts * Is) * 2);
  L.hs = take((Tk * (I / 32) + Ts * (Is / 32)) * 8);   // (S1, S2) per 32-column half
  L.yslot = take((Tk + Ts) * H * 4);
  L.xn = take((c.flags & MOE_F_RMSNORM) ? T * H * 4 : 0);
  L.cache = take(kCacheBytes);
  L.total = o;
  return L;
}

}  // namespace qreb

static int check_config(const moe_config* c) {
  if (!c || c->struct_size != sizeof(moe_config)) return MOE_EINVAL;
  if (c->group != 64) return MOE_EUNSUPPORTED;
  if (c->hidden < 64 || c->hidden > 16384 || c->hidden % 64) return MOE_EUNSUPPORTED;
  if (c->inter < 64 || c->inter > 16384 || c->inter % 64) return MOE_EUNSUPPORTED;
  if (c->n_experts < 1 || c->n_experts > kMaxExperts) return MOE_EUNSUPPORTED;
  if (c->top_k < 1 || c->top_k > c->n_experts || c->top_k > kMaxTopK) return MOE_EUNSUPPORTED;
  if (c->max_tokens < 1 || c->max_tokens > 65536) return MOE_EUNSUPPORTED;
  if (c->flags & ~(MOE_F_SHARED | MOE_F_RMSNORM | MOE_F_VERIFY)) return MOE_EUNSUPPORTED;
  if (c->flags & MOE_F_SHARED) {
    if (c->shared_inter < 64 || c->shared_inter > 16384 || c->shared_inter % 64)
      return MOE_EUNSUPPORTED;
  }
  if (c->device < 0) return MOE_EINVAL;
  return MOE_OK;
}

static int fail(moe_ctx* ctx, int code, const char* fmt, ...) {
  if (ctx) {
    char buf[512];
    va_list ap;
    va_start(ap, fmt);
    vsnprintf(buf, sizeof buf, fmt, ap);
    va_end(ap);
    ctx->err = buf;
  }
  return code;
}

static int hip_fail(moe_ctx* ctx, hipError_t e, const char* what) {
  return fail(ctx, MOE_EHIP, "%s: %s", what, hipGetErrorString(e));
}

extern "C" {

uint64_t moe_workspace_bytes(const moe_config* cfg) {
  if (check_config(cfg) != MOE_OK) return 0;
  return ws_layout(*cfg).total;
}

int moe_open(const moe_config* cfg, moe_ctx** out) {
  if (!out) return MOE_EINVAL;
  const int rc = check_config(cfg);
  if (rc != MOE_OK) return rc;
  int ndev = 0;
  if (hipGetDeviceCount(&ndev) != hipSuccess || cfg->device >= ndev) return MOE_EHIP;
  moe_ctx* c = new moe_ctx();
  c->cfg = *cfg;
  LayerDev& d = c->d;
  memset(&d, 0, sizeof d);
  d.H = cfg->hidden;
  d.E = cfg->n_experts;
  d.Epad = (cfg->n_experts + 63) / 64 * 64;
  d.k = cfg->top_k;
  d.I = cfg->inter;
  d.has_shared = (cfg->flags & MOE_F_SHARED) ? 1 : 0;
  d.Is = d.has_shared ? cfg->shared_inter : 0;
  d.rmsnorm = (cfg->flags & MOE_F_RMSNORM) ? 1 : 0;
  d.max_tokens = cfg->max_tokens;
  // Experts with 2 or 3 rows stream at hidden 2816 (16 tokens: 77.7 against
  // 83 us per forward when they take 32-row matrix-core tiles).  At hidden
  // 7168 the streaming path (fp16 token rows, one product per row) beats the
  // tiles for 2-row experts: 64 tokens 2003 against 2165 us per forward
  // (3 or more rows on the tiles), the 256-token stack 7.79 against 7.97 ms.
  d.mfma_min_rows = cfg->hidden >= 4096 ? 3 : 4;
  // 128-row tiles from 24 rows: the 256-token stack 7.03 against 7.08 ms per
  // step (eager; 20, 28 and 32 rows all slower), 16 x 128 prefill chunks
  // 2.25-2.27 against 2.29 ms, the 64-token layer and the 2048-token grouped
  // prefill within noise.
  d.wide_min_rows = 24;
  d.L = ws_layout(*cfg);
  if (hipSetDevice(cfg->device) != hipSuccess ||
      hipStreamCreateWithFlags(&c->side, hipStreamNonBlocking) != hipSuccess ||
      hipEventCreateWithFlags(&c->fork, hipEventDisableTiming) != hipSuccess ||
      hipEventCreateWithFlags(&c->join, hipEventDisableTiming) != hipSuccess) {
    moe_close(c);
    return MOE_EHIP;
  }
  int n_cu = 0;
  if (hipDeviceGetAttribute(&n_cu, hipDeviceAttributeMultiprocessorCount, cfg->device) != hipSuccess ||
      n_cu <= 0) {
    moe_close(c);
    return MOE_EHIP;
  }
  d.n_cu = n_cu;
  // 32-row tiles split by columns once the most tiles a batch can have give
  // four workgroups per CU that way (stack of 256 tokens at hidden 7168:
  // 7.82 against 8.10 ms per step); fewer keep the K split, four times the
  // workgroups (16 tokens at hidden 2816: 80 against 104 us)
  d.narrow_cs_min_wgs = 4 * n_cu;
  if (noalloc_scratch(cfg->device, &c->scratch) != hipSuccess) {
    moe_close(c);
    return MOE_EHIP;
  }
  *out = c;
  return MOE_OK;
}

int moe_set_weights(moe_ctx* ctx, const moe_weights* w, void* stream) {
  if (!ctx) return MOE_EINVAL;
  if (ctx->pf_pending) {   // a prefetch may still be copying into the old slots
    (void)hipEventSynchronize(ctx->pf_done);
    ctx->pf_pending = false;
  }
  ctx->has_weights = false;
  const moe_config& c = ctx->cfg;
  if (!w || w->struct_size != sizeof(moe_weights))
    return fail(ctx, MOE_EINVAL, "moe_weights is NULL or has the wrong struct_size");
  if (!w->router || !w->bank)
    return fail(ctx, MOE_EINVAL, "router and bank must be non-NULL");
  if (!w->workspace && w->workspace_bytes != 0)
    return fail(ctx, MOE_EINVAL, "workspace is NULL but workspace_bytes is not 0");
  if (((uintptr_t)w->workspace & 255) || ((uintptr_t)w->router & 15) || ((uintptr_t)w->bank & 255))
    return fail(ctx, MOE_EINVAL, "workspace and bank must be 256-byte aligned, router 16-byte");
  if (ctx->d.has_shared != (w->shared_record != nullptr))
    return fail(ctx, MOE_EINVAL, "shared_record must be given iff the config has MOE_F_SHARED");
  if (w->shared_record && ((uintptr_t)w->shared_record & 255))
    return fail(ctx, MOE_EINVAL, "shared_record must be 256-byte aligned");
  if (w->record_stride == 0 || w->record_stride % 4096)
    return fail(ctx, MOE_EINVAL, "record_stride must be a positive multiple of 4096");
  if (w->workspace && w->workspace_bytes < ctx->d.L.total)
    return fail(ctx, MOE_ENOMEM, "workspace has %llu bytes, needs %llu",
                (unsigned long long)w->workspace_bytes, (unsigned long long)ctx->d.L.total);
  hipError_t e = hipSetDevice(c.device);
  if (e != hipSuccess) return hip_fail(ctx, e, "hipSetDevice");
  hipStream_t s = static_cast<hipStream_t>(stream);
  std::vector<uint8_t> hdr((size_t)c.n_experts * 256);
  const void* bank_dev = device_view(w->bank);
  if (!bank_dev)
    return fail(ctx, MOE_EINVAL, "bank is neither device memory nor pinned, mapped host memory");
  e = hipMemcpy2DAsync(hdr.data(), 256, w->bank, w->record_stride, 256, c.n_experts,
                       hipMemcpyDefault, s);
  if (e != hipSuccess) return hip_fail(ctx, e, "copying record headers");
  std::vector<uint8_t> shdr(256);
  if (w->shared_record) {
    e = hipMemcpyAsync(shdr.data(), w->shared_record, 256, hipMemcpyDeviceToHost, s);
    if (e != hipSuccess) return hip_fail(ctx, e, "copying the shared record header");
  }
  e = hipStreamSynchronize(s);
  if (e != hipSuccess) return hip_fail(ctx, e, "hipStreamSynchronize");
  for (int i = 0; i < c.n_experts; ++i) {
    const int rc = moe_check_record_header(hdr.data() + (size_t)i * 256, 256, &c, i,
                                           w->record_stride);
    if (rc != MOE_OK) return fail(ctx, rc, "record %d failed header validation", i);
  }
  if (w->shared_record) {
    const int rc = moe_check_record_header(shdr.data(), 256, &c, -1, UINT64_MAX);
    if (rc != MOE_OK) return fail(ctx, rc, "shared record failed header validation");
  }
  if (c.flags & MOE_F_VERIFY) {
    // payload checksums: every record must carry one, and the GPU's CRC of
    // its payload must equal it
    auto rd32 = [](const uint8_t* p) { uint32_t v; memcpy(&v, p, 4); return v; };
    auto check = [&](const uint8_t* dev, const uint8_t* h, int n, uint64_t stride,
                     const char* what) -> int {
      for (int i = 0; i < n; ++i)
        if (rd32(h + (size_t)i * 256 + 68) != 1u)
          return fail(ctx, MOE_EBADRECORD, "%s %d carries no payload checksum", what, i);
      std::vector<uint32_t> got(n);
      uint64_t off, end;
      memcpy(&off, h + 32, 8);
      memcpy(&end, h + 56, 8);
      hipError_t e2 = crc32_ranges(dev, stride, off, end - off, n,
                                   reinterpret_cast<uint32_t*>(ctx->scratch),
                                   kNoallocScratchBytes / 4, got.data(), s);
      if (e2 != hipSuccess) return hip_fail(ctx, e2, "payload checksums");
      for (int i = 0; i < n; ++i) {
        const uint32_t want = rd32(h + (size_t)i * 256 + 64);
        if (got[i] != want)
          return fail(ctx, MOE_EBADRECORD, "%s %d: payload crc32 %08x, header says %08x", what, i,
                      got[i], want);
      }
      return MOE_OK;
    };
    int rc = check(static_cast<const uint8_t*>(bank_dev), hdr.data(), c.n_experts, w->record_stride,
                   "record");
    if (rc == MOE_OK && w->shared_record)
      rc = check(static_cast<const uint8_t*>(w->shared_record), shdr.data(), 1, 0, "shared record");
    if (rc != MOE_OK) return rc;
  }
  LayerDev& d = ctx->d;
  d.router = static_cast<const uint8_t*>(w->router);
  d.router_bias = w->router_bias;
  d.bank = static_cast<const uint8_t*>(bank_dev);
  d.stride = w->record_stride;
  d.slot_of = nullptr;                       // any expert cache is unbound with the old bank
  d.cache_src = nullptr;
  d.cache_slots = 0;
  {
    uint64_t end;
    memcpy(&end, hdr.data() + 56, 8);
    d.rec_bytes = end;
  }
  d.shared = static_cast<const uint8_t*>(w->shared_record);
  d.ws = static_cast<uint8_t*>(w->workspace);
  if (d.ws) {
    e = launch_ws_init(d, s);
    if (e != hipSuccess) return hip_fail(ctx, e, "workspace init");
  }
  ctx->has_weights = true;
  ctx->err.clear();
  return MOE_OK;
}

static int check_forward(moe_ctx* ctx, const void* x, int32_t x_dtype, int32_t n_tokens,
                         const void* out) {
  if (!ctx) return MOE_EINVAL;
  if (!ctx->has_weights) return fail(ctx, MOE_ESTATE, "no weights bound");
  if (x_dtype != MOE_BF16 && x_dtype != MOE_F32) return fail(ctx, MOE_EINVAL, "bad x dtype");
  if (n_tokens < 0 || n_tokens > ctx->cfg.max_tokens)
    return fail(ctx, MOE_EINVAL, "n_tokens %d outside [0, %d]", n_tokens, ctx->cfg.max_tokens);
  if (n_tokens > 0 && (!x || !out)) return fail(ctx, MOE_EINVAL, "x and output must be non-NULL");
  // the kernels read x rows in 16-byte pieces (rows are H * 2 or H * 4 bytes,
  // multiples of 128, so every row is then aligned as well)
  if (n_tokens > 0 && ((uintptr_t)x & 15)) return fail(ctx, MOE_EINVAL, "x must be 16-byte aligned");
  return MOE_OK;
}

// One forward on the workspace d.ws points at (the bound one, or the static
// scratch for moe_forward_noalloc).  Arguments are already checked.
static int forward_impl(moe_ctx* ctx, const LayerDev& d, const void* x, int32_t x_dtype,
                        int32_t n_tokens, float* y, const float* residual, int32_t* ids_out,
                        float* p_out, moe_ctx* next, hipStream_t s) {
  // Timing events are recorded only on a stream that is not being captured
  // into a graph (inside a capture an event record would only be a dependency).
  hipStreamCaptureStatus cap = hipStreamCaptureStatusNone;
  if (ctx->prof_calls < ctx->prof_max) (void)hipStreamIsCapturing(s, &cap);
  const bool prof = ctx->prof_calls < ctx->prof_max && cap == hipStreamCaptureStatusNone;
  const int call = ctx->prof_calls;
  auto mark = [&](int slot, int end, hipStream_t st) {
    if (!prof || !((ctx->prof_mask >> slot) & 1u)) return;
    (void)hipEventRecord(ctx->ev[((size_t)call * MOE_PROFILE_SLOTS + slot) * 2 + end], st);
    if (end) ctx->launched[(size_t)call * MOE_PROFILE_SLOTS + slot] = 1;
  };
  hipError_t e = hipSuccess;
  // a prefetch into this context's cache (issued by the previous layer's
  // lookahead) must land before this forward plans its cache
  if (ctx->pf_pending) {
    if ((e = hipStreamWaitEvent(s, ctx->pf_done, 0)) != hipSuccess)
      return hip_fail(ctx, e, "waiting for the prefetch");
    ctx->pf_pending = false;
  }
  mark(0, 0, s);
  const void* xin = x;
  int f32 = x_dtype == MOE_F32;
  if (d.rmsnorm) {   // the layer (and a lookahead router) sees the normalized rows
    e = launch_rmsnorm(d, x, f32, n_tokens, s);
    if (e != hipSuccess) return hip_fail(ctx, e, "rmsnorm launch");
    xin = d.ws + d.L.xn;
    f32 = 1;
  }
  e = launch_router(d, xin, f32, n_tokens, 0, nullptr, ids_out, p_out, s);
  if (e != hipSuccess) return hip_fail(ctx, e, "router launch");
  mark(0, 1, s);
  const int max_sel = n_tokens * d.k < d.E ? n_tokens * d.k : d.E;
  if (d.slot_of) {   // the experts of this forward into the cache
    mark(6, 0, s);
    if ((e = launch_cache_plan(d, 0, 0, 0, s)) != hipSuccess ||
        (e = launch_cache_fill(d, 0, max_sel, s)) != hipSuccess)
      return hip_fail(ctx, e, "expert cache");
    mark(6, 1, s);
  }
  // The next layer's router on this input ("one residual ahead"): its
  // prediction orders that layer's work and, with a cache there, prefetches
  // its experts on that context's copy stream while this layer computes.
  // It reads x before the combine writes y, so y may alias x.  Without a
  // prefetch to start it runs after this layer's streaming launches, beside
  // the longer wide matrix-core path, instead of ahead of the experts (the
  // stack: about 40 us per layer off the critical path).
  const bool la_early = next && next->d.slot_of && (next->cache_flags & MOE_CACHE_PREFETCH);
  if (la_early) {
    e = launch_router(next->d, xin, f32, n_tokens, 2, nullptr, nullptr, nullptr, s);
    if (e != hipSuccess) return hip_fail(ctx, e, "lookahead router launch");
    {
      const int nmax = n_tokens * next->d.k < next->d.E ? n_tokens * next->d.k : next->d.E;
      if ((e = hipEventRecord(next->pf_done, s)) != hipSuccess ||
          (e = hipStreamWaitEvent(next->copy, next->pf_done, 0)) != hipSuccess ||
          (e = launch_cache_plan(next->d, 1, n_tokens * next->d.k, (int)((next->cache_flags >> 8) & 0xffu),
                                 next->copy)) != hipSuccess ||
          (e = launch_cache_fill(next->d, 1, nmax, next->copy)) != hipSuccess ||
          (e = hipEventRecord(next->pf_done, next->copy)) != hipSuccess)
        return hip_fail(ctx, e, "lookahead prefetch");
      next->pf_pending = true;
    }
  }
  // Wide matrix-core work (experts with many rows) runs concurrently with
  // the streaming launches, which also carry the narrow matrix-core tiles;
  // the two touch disjoint slots.  The wide launches stay on the caller's
  // stream and the streaming ones move to the context's side stream behind
  // a fork: the wide gate/up launch, the longer path, then reaches the CUs
  // first (the 256-token stack at hidden 7168: 7.40 against 7.49 ms per
  // step).  Decode-sized batches need no wide work and so no fork or join.
  const bool mf = mfma_needed(d, n_tokens);
  hipStream_t gs = s;   // the streaming launches' stream
  if (mf) {
    gs = ctx->side;
    if ((e = hipEventRecord(ctx->fork, s)) != hipSuccess ||
        (e = hipStreamWaitEvent(gs, ctx->fork, 0)) != hipSuccess)
      return hip_fail(ctx, e, "forking the streaming stream");
    mark(3, 0, s);
    e = launch_mfma_up(d, n_tokens, s);
    if (e != hipSuccess) return hip_fail(ctx, e, "matrix-core gate/up launch");
    mark(3, 1, s);
    mark(4, 0, s);
    e = launch_mfma_down(d, n_tokens, s);
    if (e != hipSuccess) return hip_fail(ctx, e, "matrix-core down launch");
    mark(4, 1, s);
  }
  mark(1, 0, gs);
  e = launch_gemv_up(d, n_tokens, gs);
  if (e != hipSuccess) return hip_fail(ctx, e, "streaming gate/up launch");
  mark(1, 1, gs);
  mark(2, 0, gs);
  e = launch_gemv_down(d, n_tokens, gs);
  if (e != hipSuccess) return hip_fail(ctx, e, "streaming down launch");
  mark(2, 1, gs);
  if (next && !la_early) {
    e = launch_router(next->d, xin, f32, n_tokens, 2, nullptr, nullptr, nullptr, gs);
    if (e != hipSuccess) return hip_fail(ctx, e, "lookahead router launch");
  }
  if (mf) {
    if ((e = hipEventRecord(ctx->join, gs)) != hipSuccess ||
        (e = hipStreamWaitEvent(s, ctx->join, 0)) != hipSuccess)
      return hip_fail(ctx, e, "joining the streaming stream");
  }
  mark(5, 0, s);
  e = launch_combine(d, n_tokens, reinterpret_cast<const float*>(d.ws + d.L.p), residual, y, s);
  if (e != hipSuccess) return hip_fail(ctx, e, "combine launch");
  mark(5, 1, s);
  if (prof) ctx->prof_calls++;
  return MOE_OK;
}

int moe_forward(moe_ctx* ctx, const void* x, int32_t x_dtype, int32_t n_tokens, float* y,
                const float* residual, int32_t* ids_out, float* p_out, moe_ctx* next,
                void* stream) {
  int rc = check_forward(ctx, x, x_dtype, n_tokens, y);
  if (rc != MOE_OK) return rc;
  if (!ctx->d.ws)
    return fail(ctx, MOE_ESTATE, "no workspace bound (this context runs moe_forward_noalloc only)");
  if (next) {
    if (next == ctx) return fail(ctx, MOE_EINVAL, "lookahead context is this context");
    if (!next->has_weights) return fail(ctx, MOE_ESTATE, "lookahead context has no weights");
    if (!next->d.ws) return fail(ctx, MOE_EINVAL, "lookahead context has no workspace bound");
    if (next->cfg.hidden != ctx->cfg.hidden || next->cfg.max_tokens < n_tokens ||
        next->d.rmsnorm != ctx->d.rmsnorm)
      return fail(ctx, MOE_EINVAL, "lookahead context does not match this layer");
  }
  if (n_tokens == 0) return MOE_OK;
  return forward_impl(ctx, ctx->d, x, x_dtype, n_tokens, y, residual, ids_out, p_out, next,
                      static_cast<hipStream_t>(stream));
}

int moe_forward_noalloc(moe_ctx* ctx, const void* x, int32_t x_dtype, int32_t n_tokens, float* y,
                        const float* residual, int32_t* ids_out, float* p_out, void* stream) {
  int rc = check_forward(ctx, x, x_dtype, n_tokens, y);
  if (rc != MOE_OK) return rc;
  if (ctx->d.slot_of)
    return fail(ctx, MOE_EINVAL, "a context with an expert cache keeps its state in its workspace");
  if (n_tokens == 0) return MOE_OK;
  // The workspace layout for exactly this batch, placed in the static scratch.
  LayerDev d = ctx->d;
  moe_config c = ctx->cfg;
  c.max_tokens = n_tokens;
  d.L = ws_layout(c);
  if (d.L.total > kNoallocScratchBytes)
    return fail(ctx, MOE_ENOMEM,
                "a forward of %d tokens needs %llu bytes of scratch; the static scratch holds %llu",
                n_tokens, (unsigned long long)d.L.total, (unsigned long long)kNoallocScratchBytes);
  if (!ctx->scratch) return fail(ctx, MOE_ESTATE, "no static scratch on this device");
  d.ws = ctx->scratch;
  hipStream_t s = static_cast<hipStream_t>(stream);
  // Another call may have left its state in the shared array: clear the
  // counters (no lookahead prediction pending) with a fill kernel.
  hipError_t e = launch_ws_init(d, s);
  if (e != hipSuccess) return hip_fail(ctx, e, "scratch init");
  return forward_impl(ctx, d, x, x_dtype, n_tokens, y, residual, ids_out, p_out, nullptr, s);
}

int moe_profile_start(moe_ctx* ctx, int32_t max_calls) {
  return moe_profile_start_slots(ctx, max_calls, 0xffu);
}

int moe_profile_start_slots(moe_ctx* ctx, int32_t max_calls, uint32_t slot_mask) {
  if (!ctx || max_calls < 1 || max_calls > 100000 || slot_mask == 0 ||
      (slot_mask >> MOE_PROFILE_SLOTS))
    return MOE_EINVAL;
  prof_clear(ctx);
  ctx->prof_mask = slot_mask;
  ctx->ev.resize((size_t)max_calls * MOE_PROFILE_SLOTS * 2);
  for (auto& e : ctx->ev) {
    // timing-only events: no system-scope fence (cache writeback and
    // invalidation) around the kernel they bracket
    hipError_t r = hipEventCreateWithFlags(&e, hipEventDisableSystemFence);
    if (r != hipSuccess) {
      e = nullptr;
      prof_clear(ctx);
      return hip_fail(ctx, r, "hipEventCreate");
    }
  }
  ctx->launched.assign((size_t)max_calls * MOE_PROFILE_SLOTS, 0);
  ctx->prof_max = max_calls;
  return MOE_OK;
}

int moe_profile_read(moe_ctx* ctx, float* avg_ms, int32_t* n_calls, int32_t n_slots) {
  if (!ctx || !avg_ms || !n_calls || n_slots < 0) return MOE_EINVAL;
  const int calls = ctx->prof_calls;
  for (int i = 0; i < n_slots; ++i) avg_ms[i] = 0.f;
  for (int slot = 0; slot < MOE_PROFILE_SLOTS && slot < n_slots; ++slot) {
    double sum = 0;
    int n = 0;
    for (int c = 0; c < calls; ++c) {
      if (!ctx->launched[(size_t)c * MOE_PROFILE_SLOTS + slot]) continue;
      hipEvent_t b = ctx->ev[((size_t)c * MOE_PROFILE_SLOTS + slot) * 2];
      hipEvent_t e = ctx->ev[((size_t)c * MOE_PROFILE_SLOTS + slot) * 2 + 1];
      hipError_t r = hipEventSynchronize(e);
      float ms = 0.f;
      if (r == hipSuccess) r = hipEventElapsedTime(&ms, b, e);
      if (r != hipSuccess) {
        prof_clear(ctx);
        return hip_fail(ctx, r, "reading kernel timing events");
      }
      sum += ms;
      ++n;
    }
    avg_ms[slot] = n ? (float)(sum / n) : 0.f;
  }
  *n_calls = calls;
  prof_clear(ctx);
  return MOE_OK;
}

int moe_router_logits(moe_ctx* ctx, const void* x, int32_t x_dtype, int32_t n_tokens,
                      float* logits, void* stream) {
  int rc = check_forward(ctx, x, x_dtype, n_tokens, logits);
  if (rc != MOE_OK) return rc;
  if (!ctx->d.ws) return fail(ctx, MOE_ESTATE, "no workspace bound");
  if (n_tokens == 0) return MOE_OK;
  const LayerDev& d = ctx->d;
  hipStream_t s = static_cast<hipStream_t>(stream);
  const void* xin = x;
  int f32 = x_dtype == MOE_F32;
  hipError_t e;
  if (d.rmsnorm) {   // the router sees what the layer sees
    e = launch_rmsnorm(d, x, f32, n_tokens, s);
    if (e != hipSuccess) return hip_fail(ctx, e, "rmsnorm launch");
    xin = d.ws + d.L.xn;
    f32 = 1;
  }
  e = launch_router(d, xin, f32, n_tokens, 1, logits, nullptr, nullptr, s);
  if (e != hipSuccess) return hip_fail(ctx, e, "router launch");
  return MOE_OK;
}

int moe_set_path_rows(moe_ctx* ctx, int32_t mfma_min_rows, int32_t wide_min_rows) {
  if (!ctx) return MOE_EINVAL;
  if (mfma_min_rows < 1 || wide_min_rows < mfma_min_rows)
    return fail(ctx, MOE_EINVAL, "need 1 <= mfma_min_rows <= wide_min_rows");
  ctx->d.mfma_min_rows = mfma_min_rows;
  ctx->d.wide_min_rows = wide_min_rows;
  return MOE_OK;
}

int moe_set_narrow_split(moe_ctx* ctx, int32_t min_workgroups) {
  if (!ctx) return MOE_EINVAL;
  if (min_workgroups < 0) return fail(ctx, MOE_EINVAL, "need min_workgroups >= 0");
  ctx->d.narrow_cs_min_wgs = min_workgroups;
  return MOE_OK;
}

void moe_close(moe_ctx* ctx) {
  if (!ctx) return;
  if (ctx->pf_pending) (void)hipEventSynchronize(ctx->pf_done);
  prof_clear(ctx);
  if (ctx->join) (void)hipEventDestroy(ctx->join);
  if (ctx->fork) (void)hipEventDestroy(ctx->fork);
  if (ctx->side) (void)hipStreamDestroy(ctx->side);
  if (ctx->pf_done) (void)hipEventDestroy(ctx->pf_done);
  if (ctx->copy) (void)hipStreamDestroy(ctx->copy);
  delete ctx;
}

const char* moe_strerror(int code) {
  switch (code) {
    case MOE_OK: return "ok";
    case MOE_EINVAL: return "invalid argument";
    case MOE_EUNSUPPORTED: return "unsupported shape or option";
    case MOE_ENOMEM: return "workspace too small";
    case MOE_EBADRECORD: return "record header failed validation";
    case MOE_ESTATE: return "call out of order (no weights bound)";
    case MOE_EHIP: return "HIP runtime error";
    default: return "unknown status";
  }
}

const char* moe_last_error(const moe_ctx* ctx) { return ctx ? ctx->err.c_str() : ""; }

int moe_set_cache(moe_ctx* ctx, void* slots, uint64_t slots_bytes, int32_t n_slots, uint32_t flags,
                  void* stream) {
  if (!ctx) return MOE_EINVAL;
  if (!ctx->has_weights) return fail(ctx, MOE_ESTATE, "no weights bound");
  LayerDev& d = ctx->d;
  if (!d.ws) return fail(ctx, MOE_ESTATE, "the expert cache keeps its state in the bound workspace");
  if (flags & ~(MOE_CACHE_PREFETCH | MOE_CACHE_PREFETCH_TOP(0xff)))
    return fail(ctx, MOE_EINVAL, "unknown cache flags");
  const uint32_t top = (flags >> 8) & 0xffu;
  if (top && (!(flags & MOE_CACHE_PREFETCH) || top > (uint32_t)d.k))
    return fail(ctx, MOE_EINVAL, "a prefetch depth needs MOE_CACHE_PREFETCH and at most k (%d)", d.k);
  hipStream_t s = static_cast<hipStream_t>(stream);
  hipError_t e = hipSetDevice(ctx->cfg.device);
  if (e != hipSuccess) return hip_fail(ctx, e, "hipSetDevice");
  // a prefetch still copying into the old slots must finish first
  if (ctx->pf_pending) {
    if ((e = hipEventSynchronize(ctx->pf_done)) != hipSuccess) return hip_fail(ctx, e, "prefetch");
    ctx->pf_pending = false;
  }
  const uint8_t* src = d.slot_of ? d.cache_src : d.bank;
  if (!slots || n_slots == 0) {   // unbind: the kernels read the bank again
    d.bank = src;
    d.slot_of = nullptr;
    d.cache_src = nullptr;
    d.cache_slots = 0;
    ctx->cache_flags = 0;
    return MOE_OK;
  }
  const int need = ctx->cfg.max_tokens * d.k < d.E ? ctx->cfg.max_tokens * d.k : d.E;
  if (n_slots < need || n_slots > d.E)
    return fail(ctx, MOE_ENOMEM,
                "%d cache slots: a forward of %d tokens may select %d experts (slots must be in "
                "[%d, %d])", n_slots, ctx->cfg.max_tokens, need, need, d.E);
  if ((uintptr_t)slots & 255) return fail(ctx, MOE_EINVAL, "slots must be 256-byte aligned");
  if (slots_bytes < (uint64_t)n_slots * d.stride)
    return fail(ctx, MOE_ENOMEM, "slots hold %llu bytes, %d records need %llu",
                (unsigned long long)slots_bytes, n_slots, (unsigned long long)n_slots * d.stride);
  hipPointerAttribute_t a;
  if (hipPointerGetAttributes(&a, slots) != hipSuccess || a.type != hipMemoryTypeDevice) {
    (void)hipGetLastError();
    return fail(ctx, MOE_EINVAL, "slots must be device memory");
  }
  if (!ctx->copy && (e = hipStreamCreateWithFlags(&ctx->copy, hipStreamNonBlocking)) != hipSuccess) {
    ctx->copy = nullptr;
    return hip_fail(ctx, e, "creating the prefetch stream");
  }
  if (!ctx->pf_done && (e = hipEventCreateWithFlags(&ctx->pf_done, hipEventDisableTiming)) != hipSuccess) {
    ctx->pf_done = nullptr;
    return hip_fail(ctx, e, "creating the prefetch event");
  }
  d.cache_src = src;
  d.cache_src_stride = d.stride;
  d.bank = static_cast<const uint8_t*>(slots);
  d.slot_of = reinterpret_cast<const int*>(d.ws + d.L.cache + kCacheSlotOf);
  d.cache_slots = n_slots;
  ctx->cache_flags = flags;
  e = launch_cache_reset(d, s);
  if (e != hipSuccess) return hip_fail(ctx, e, "cache reset");
  return MOE_OK;
}

int moe_cache_stats(moe_ctx* ctx, uint64_t* out, int32_t n, void* stream) {
  if (!ctx || !out || n < 0) return MOE_EINVAL;
  if (!ctx->d.slot_of) return fail(ctx, MOE_ESTATE, "no expert cache");
  const int m = n < kCacheStats ? n : kCacheStats;
  hipStream_t s = static_cast<hipStream_t>(stream);
  hipError_t e = hipSuccess;
  if (ctx->pf_pending) e = hipStreamWaitEvent(s, ctx->pf_done, 0);
  if (e == hipSuccess)
    e = hipMemcpyAsync(out, ctx->d.ws + ctx->d.L.cache + kCacheStatsOff, (size_t)m * 8,
                       hipMemcpyDeviceToHost, s);
  if (e == hipSuccess) e = hipStreamSynchronize(s);
  if (e != hipSuccess) return hip_fail(ctx, e, "reading the cache counters");
  for (int i = m; i < n; ++i) out[i] = 0;
  return MOE_OK;
}

uint64_t moe_rvq_workspace_bytes(int32_t n_tokens, int32_t k_cols, int32_t rows, int32_t n_mats) {
  if (n_tokens < 1 || n_tokens > 65535 || k_cols < 64 || k_cols % 64 || rows < 64 || rows % 64 ||
      n_mats < 1)
    return 0;
  return rvq_workspace(n_tokens, k_cols, rows, n_mats);   // 0 past the launch limits
}

int moe_rvq_gemv(const void* x, int32_t x_dtype, int32_t n_tokens, int32_t k_cols,
                 const void* mats, uint64_t mat_stride, int32_t n_mats, int32_t rows,
                 const void* codebooks, float* y, void* workspace, uint64_t workspace_bytes,
                 void* stream) {
  if (n_tokens == 0) return MOE_OK;
  const uint64_t need = moe_rvq_workspace_bytes(n_tokens, k_cols, rows, n_mats);
  if (need == 0 || n_tokens < 0 || (x_dtype != MOE_BF16 && x_dtype != MOE_F32)) return MOE_EINVAL;
  if (!x || !mats || !codebooks || !y || !workspace) return MOE_EINVAL;
  if (((uintptr_t)mats & 15) || (mat_stride & 15) ||
      (n_mats > 1 && mat_stride < (uint64_t)(rows / 64) * (k_cols / 64) * 1536))
    return MOE_EINVAL;
  if (((uintptr_t)workspace & 255) || ((uintptr_t)codebooks & 15) || ((uintptr_t)x & 3) ||
      ((uintptr_t)y & 3))
    return MOE_EINVAL;
  if (workspace_bytes < need) return MOE_ENOMEM;
  const hipError_t e = launch_rvq_gemv(x, x_dtype == MOE_F32, n_tokens, k_cols,
                                       static_cast<const uint8_t*>(mats), mat_stride, n_mats, rows,
                                       static_cast<const uint16_t*>(codebooks), y,
                                       static_cast<uint8_t*>(workspace),
                                       static_cast<hipStream_t>(stream));
  return e == hipSuccess ? MOE_OK : MOE_EHIP;
}

int moe_crc32(const void* dev_bytes, uint64_t n_bytes, uint32_t* crc_out, void* stream) {
  if (!crc_out) return MOE_EINVAL;
  if (n_bytes == 0) {   // the CRC of no bytes
    *crc_out = 0;
    return MOE_OK;
  }
  if (!dev_bytes || ((uintptr_t)dev_bytes & 15)) return MOE_EINVAL;
  int dev = 0;
  uint8_t* tmp = nullptr;
  if (hipGetDevice(&dev) != hipSuccess || noalloc_scratch(dev, &tmp) != hipSuccess) return MOE_EHIP;
  const hipError_t e = crc32_ranges(static_cast<const uint8_t*>(dev_bytes), 0, 0, n_bytes, 1,
                                    reinterpret_cast<uint32_t*>(tmp), kNoallocScratchBytes / 4,
                                    crc_out, static_cast<hipStream_t>(stream));
  return e == hipSuccess ? MOE_OK : MOE_EHIP;
}

int moe_debug_dequant(const void* tiles, int32_t bits, int32_t rows, int32_t cols, float* out,
                      void* stream) {
  if (!tiles || !out || (bits != 4 && bits != 8) || rows <= 0 || cols <= 0 || rows % 64 ||
      cols % 64)
    return MOE_EINVAL;
  hipError_t e = launch_debug_dequant(tiles, bits, rows, cols, out,
                                      static_cast<hipStream_t>(stream));
  return e == hipSuccess ? MOE_OK : MOE_EHIP;
}

}  // extern "C"
