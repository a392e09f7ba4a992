// Host runtime of the tattn C ABI: validation (pure host), workspace layout,
// launch sequencing on the caller's stream and HIP-error -> status mapping.
#include <hip/hip_runtime.h>

#include <algorithm>
#include <cmath>
#include <cstdarg>
#include <cstdio>
#include <cstring>
#include <mutex>
#include <string>
#include <vector>

#include "../../include/tattn.h"
#include "tattn_device.hpp"
#include "tattn_internal.hpp"

namespace tattn {

static thread_local std::string g_err;

static tattn_status fail(tattn_status st, const char* fmt, ...) __attribute__((format(printf, 2, 3)));
static tattn_status fail(tattn_status st, const char* fmt, ...) {
  char buf[512];
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(buf, sizeof(buf), fmt, ap);
  va_end(ap);
  g_err = buf;
  return st;
}
static tattn_status ok() {
  g_err.clear();
  return TATTN_OK;
}
static tattn_status hip_fail(hipError_t e, const char* what) {
  return fail(TATTN_E_HIP, "%s: %s", what, hipGetErrorString(e));
}

Dims make_dims(const tattn_config& c) {
  Dims d;
  d.B = c.batch;
  d.H = c.heads;
  d.BH = c.batch * c.heads;
  d.N = c.seq_len;
  d.D = c.head_dim;
  d.Bq = c.block_q;
  d.Bk = c.block_k;
  d.Nq = (c.seq_len + c.block_q - 1) / c.block_q;
  d.Nk = (c.seq_len + c.block_k - 1) / c.block_k;
  d.NkC = (d.Nk + 63) / 64;
  d.sb = c.stride_b;
  d.sh = c.stride_h;
  d.sn = c.stride_n;
  return d;
}

Layout make_layout(const Dims& d, int entropy_samples, bool moments, bool skim, bool refine) {
  Layout L;
  size_t off = 0;
  auto take = [&](size_t bytes) {
    const size_t at = off;
    off += (bytes + kAlign - 1) / kAlign * kAlign;
    return at;
  };
  const size_t BH = d.BH, Nq = d.Nq, Nk = d.Nk, D = d.D, Bk = d.Bk;
  const size_t S = std::max(1, std::min(entropy_samples, d.Nq));
  L.qbar = take(BH * Nq * D * 4);
  L.kbar = take(BH * Nk * D * 4);
  L.vbar = take(BH * Nk * D * 4);
  L.sq = take(BH * Nq * 4);
  L.iq = take(BH * Nq * 4);
  L.sk = take(BH * Nk * 4);
  L.sv = take(BH * Nk * 4);
  {
    Slab& sl = L.sl;
    size_t o = 0;
    auto sub = [&](size_t bytes) {
      const size_t at = o;
      o += (bytes + kAlign - 1) / kAlign * kAlign;
      return at;
    };
    sl.v8t = sub(Nk * Bk * D);
    sl.vlow = sub(Bk < 64 ? Nk * Bk * D * 2 : 0);
    sl.k8 = sub(Nk * Bk * D);
    sl.kbhi = sub(Nk * D * 2);
    sl.kblo = sub(Nk * D * 2);
    sl.vbarT = sub((size_t)d.NkC * 64 * D * 2);
    // MXFP4 rows are made per 64-row group of the sequence
    const size_t rows64 = (size_t)(d.N + 63) / 64 * 64;
    const size_t k4n = skim || refine ? rows64 : 0, k4rn = refine ? rows64 : 0;
    sl.k4 = sub(k4n * D / 2);
    sl.k4s = sub(k4n * D / 32);
    sl.k4r = sub(k4rn * D / 2);
    sl.k4rs = sub(k4rn * D / 32);
    sl.bytes = o;
  }
  L.slab = take(BH * L.sl.bytes);
  L.S = take(BH * Nq * Nk * 8);
  L.p = take(BH * Nq * Nk * 4);
  L.tiers = take(BH * Nq * Nk);
  L.lists = take(BH * Nq * Nk * 2);
  L.counts = take(BH * Nq * 4 * 4);
  L.order = take(BH * Nq * 4);
  L.ent = take(BH * S * 8);
  L.kh = take(BH * 4);
  L.rh = take(BH * 8);
  const size_t mq = moments ? BH * Nq : 0, mk = moments ? BH * Nk : 0;
  L.q2 = take(mq * D * 4);
  L.m2q = take(mq * 4);
  L.kvar = take(mk * D * 4);
  L.m2k = take(mk * 4);
  L.vvar = take(mk * 4);
  L.m2v = take(mk * 4);
  L.vnorm = take(mk * 4);
  L.s2 = take(mq * Nk * 8);
  L.flag = take(16);
  L.total = off;
  return L;
}

static bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15) == 0; }

// The SKIM tier is on for a positive tau_skim in THRESHOLD, EXTERNAL and
// PRICE modes.
static bool skim_on(const tattn_config& c) {
  return c.tau_skim > 0.0f && c.mode != TATTN_MODE_ALL_FULL;
}
// The refined low tier: LOW tiles score on MXFP4 copies with residual correction.
static bool refine_on(const tattn_config& c) { return c.low_refine == 1; }
static Layout layout_of(const tattn_config& c) {
  return make_layout(make_dims(c), c.entropy_samples, c.mode == TATTN_MODE_PRICE, skim_on(c), refine_on(c));
}

// Most tiles a row can keep (FULL, LOW or SKIM) under the config's rule:
// ADAPTIVE keeps the top k_h <= ceil(keep_max * Nk) (the same float64 product
// the router rounds up) plus the diagonal blocks, THRESHOLD with top-k keeps
// top_k plus the diagonal; otherwise every tile may be kept.  The fused kernel
// sizes the row's list in LDS by it.
static int list_cap(const tattn_config& c, const Dims& d) {
  const int64_t ndiag = d.Bq / d.Bk + 1;
  int64_t cap = d.Nk;
  if (c.mode == TATTN_MODE_ADAPTIVE && !skim_on(c))   // (SKIM tiles lie outside the kept ones)
    cap = std::min<int64_t>(cap, (int64_t)std::ceil((double)c.keep_max * (double)d.Nk) + ndiag);
  else if (c.mode == TATTN_MODE_THRESHOLD && c.top_k > 0)
    cap = std::min<int64_t>(cap, (int64_t)c.top_k + ndiag);
  return (int)cap;
}

static tattn_status validate(const tattn_config* c) {
  if (!c) return fail(TATTN_E_INVALID, "config is NULL");
  if (c->batch < 1 || c->heads < 1 || c->seq_len < 1)
    return fail(TATTN_E_INVALID, "batch, heads and seq_len must be >= 1 (got %d, %d, %d)", c->batch, c->heads,
                c->seq_len);
  if (c->head_dim < 1 || c->block_q < 1 || c->block_k < 1)
    return fail(TATTN_E_INVALID, "head_dim, block_q and block_k must be >= 1");
  if (c->head_dim != 64 && c->head_dim != 128)
    return fail(TATTN_E_UNSUPPORTED, "head_dim %d not supported (64 or 128)", c->head_dim);
  const int bk = c->block_k;
  if ((bk != 64 && bk != 16 && bk != 8 && bk != 4 && bk != 2 && bk != 1) || (c->block_q != 64 && c->block_q != 128))
    return fail(TATTN_E_UNSUPPORTED, "tile %dx%d not supported (block_q 64 or 128, block_k 64, 16, 8, 4, 2 or 1)",
                c->block_q, c->block_k);
  if (c->mode < 0 || c->mode > 4) return fail(TATTN_E_INVALID, "mode %d out of range", c->mode);
  if (c->mode == TATTN_MODE_PRICE && (!std::isfinite(c->price) || c->price < 0.0f))
    return fail(TATTN_E_INVALID, "price must be finite and >= 0 (got %g)", c->price);
  if (!std::isfinite(c->tau_hi) || !std::isfinite(c->tau_lo) || c->tau_lo < 0.0f || c->tau_lo > c->tau_hi)
    return fail(TATTN_E_INVALID, "thresholds need 0 <= tau_lo <= tau_hi (got %g, %g)", c->tau_lo, c->tau_hi);
  if (!std::isfinite(c->tau_skim) || c->tau_skim < 0.0f)
    return fail(TATTN_E_INVALID, "tau_skim must be finite and >= 0 (got %g)", c->tau_skim);
  if (c->mode == TATTN_MODE_THRESHOLD && c->tau_skim > c->tau_lo)
    return fail(TATTN_E_INVALID, "tau_skim needs 0 <= tau_skim <= tau_lo (got %g, tau_lo %g)", c->tau_skim, c->tau_lo);
  if (c->low_refine != 0 && c->low_refine != 1) return fail(TATTN_E_INVALID, "low_refine must be 0 or 1 (got %d)", c->low_refine);
  if (refine_on(*c) && skim_on(*c))
    return fail(TATTN_E_UNSUPPORTED, "the refined low tier and the SKIM tier are not combined");
  const int64_t nq = (c->seq_len + (int64_t)c->block_q - 1) / c->block_q;
  const int64_t nk = (c->seq_len + (int64_t)c->block_k - 1) / c->block_k;
  if (c->top_k < 0 || c->top_k > nk) return fail(TATTN_E_INVALID, "top_k %d outside [0, %lld]", c->top_k, (long long)nk);
  if (c->mode == TATTN_MODE_ADAPTIVE) {
    if (!(c->keep_min > 0.0f) || !(c->keep_max >= c->keep_min) || !(c->keep_max <= 1.0f))
      return fail(TATTN_E_INVALID, "adaptive mode needs 0 < keep_min <= keep_max <= 1");
    if (!(c->full_frac > 0.0f) || !(c->full_frac <= 1.0f))
      return fail(TATTN_E_INVALID, "adaptive mode needs 0 < full_frac <= 1");
    if (c->entropy_samples < 1) return fail(TATTN_E_INVALID, "entropy_samples must be >= 1");
  }
  if (c->in_dtype != TATTN_BF16) {
    if (c->in_dtype == TATTN_FP32) return fail(TATTN_E_UNSUPPORTED, "fp32 inputs are not supported (bf16 only)");
    return fail(TATTN_E_INVALID, "in_dtype %d unknown", c->in_dtype);
  }
  if (c->out_dtype != TATTN_BF16 && c->out_dtype != TATTN_FP32)
    return fail(TATTN_E_INVALID, "out_dtype %d unknown", c->out_dtype);
  if (c->stride_n < c->head_dim || c->stride_h < 1 || c->stride_b < 1)
    return fail(TATTN_E_INVALID, "strides must be positive with stride_n >= head_dim");
  if ((c->stride_n % 8) || (c->stride_h % 8) || (c->stride_b % 8))
    return fail(TATTN_E_INVALID, "strides must be multiples of 8 elements (16-byte rows)");
  if (nk > kMaxNk) return fail(TATTN_E_UNSUPPORTED, "%lld key blocks exceed the limit of %d", (long long)nk, kMaxNk);
  if ((int64_t)c->batch * c->heads * nq > 0x7fffffffLL || (int64_t)c->batch * c->heads * nk > 0x7fffffffLL)
    return fail(TATTN_E_UNSUPPORTED, "problem too large for one launch");
  // blocks below 64 keys address a head's K and V rows with 32-bit byte offsets
  if (c->block_k != 64 && (int64_t)c->seq_len * c->stride_n * 2 > 0x7fffffffLL)
    return fail(TATTN_E_UNSUPPORTED, "seq_len x stride_n too large for %d-key blocks", c->block_k);
  return ok();
}

// ---- static scratch of tattn_attention_static: a file-scope device array
// (one per GPU, held until the process ends) whose device address is taken
// once per device with hipGetSymbolAddress; host code uses only that address.
constexpr size_t kStaticScratchBytes = size_t(64) << 20;
static __device__ __align__(256) unsigned char scratch[kStaticScratchBytes];

constexpr int kMaxDevices = 64;
static std::mutex g_scratch_mu;
static void* g_scratch_ptr[kMaxDevices];

// The current device's address of `scratch` (looked up on its first use on
// that device, with that device current).
static tattn_status static_scratch(void** out) {
  int dev = -1;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return hip_fail(e, "hipGetDevice");
  if (dev < 0 || dev >= kMaxDevices) return fail(TATTN_E_UNSUPPORTED, "device %d beyond the %d supported", dev, kMaxDevices);
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (!g_scratch_ptr[dev]) {
    void* ptr = nullptr;
    e = hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch));
    if (e != hipSuccess) return hip_fail(e, "hipGetSymbolAddress(scratch)");
    if (!ptr || reinterpret_cast<uintptr_t>(ptr) % kAlign)
      return fail(TATTN_E_HIP, "static scratch address %p is not 256-byte aligned", ptr);
    g_scratch_ptr[dev] = ptr;
  }
  *out = g_scratch_ptr[dev];
  return TATTN_OK;
}

}  // namespace tattn

using namespace tattn;

struct tattn_plan_s {
  tattn_config cfg;
  Dims d;
  Layout L;
  unsigned char* ws;
  const void* k;
  const void* v;
  bool has_tiers;
};

extern "C" {

tattn_status tattn_validate(const tattn_config* cfg) { return validate(cfg); }

tattn_status tattn_workspace_bytes(const tattn_config* cfg, size_t* bytes) {
  tattn_status st = validate(cfg);
  if (st != TATTN_OK) return st;
  if (!bytes) return fail(TATTN_E_INVALID, "bytes is NULL");
  *bytes = layout_of(*cfg).total;
  return ok();
}

static RouterArgs router_args(const tattn_plan_s* p) {
  RouterArgs r;
  r.ws = p->ws;
  r.L = p->L;
  r.d = p->d;
  r.mode = p->cfg.mode;
  r.tau_hi = p->cfg.tau_hi;
  r.tau_lo = p->cfg.tau_lo;
  r.top_k = p->cfg.top_k;
  r.keep_min = p->cfg.keep_min;
  r.keep_max = p->cfg.keep_max;
  r.full_frac = p->cfg.full_frac;
  r.samples = std::max(1, p->cfg.entropy_samples);
  r.price = p->cfg.price;
  r.tau_skim = skim_on(p->cfg) ? p->cfg.tau_skim : 0.0f;
  return r;
}

// Fill *p and launch the plan's kernels (pooling, then routing unless
// EXTERNAL) into `workspace`; the caller has validated cfg and the workspace.
static tattn_status plan_into(tattn_plan_s* p, const tattn_config* cfg, const void* q, const void* k, const void* v,
                              void* workspace, void* stream) {
  p->cfg = *cfg;
  p->d = make_dims(*cfg);
  p->L = layout_of(*cfg);
  p->ws = static_cast<unsigned char*>(workspace);
  p->k = k;
  p->v = v;
  p->has_tiers = cfg->mode != TATTN_MODE_EXTERNAL;
  hipStream_t s = static_cast<hipStream_t>(stream);
  PoolArgs pa{static_cast<const uint16_t*>(q), static_cast<const uint16_t*>(k), static_cast<const uint16_t*>(v),
              p->ws, p->L, p->d, cfg->mode == TATTN_MODE_PRICE ? 1 : 0, skim_on(*cfg) || refine_on(*cfg) ? 1 : 0,
              refine_on(*cfg) ? 1 : 0};
  hipError_t e = launch_pool(pa, s);
  if (e != hipSuccess) return hip_fail(e, "pool kernel launch");
  if (cfg->mode != TATTN_MODE_EXTERNAL) {
    e = launch_router(router_args(p), s);
    if (e != hipSuccess) return hip_fail(e, "router kernel launch");
  }
  return ok();
}

tattn_status tattn_plan(const tattn_config* cfg, const void* q, const void* k, const void* v, void* workspace,
                        size_t workspace_bytes, void* stream, tattn_plan_t* out) {
  tattn_status st = validate(cfg);
  if (st != TATTN_OK) return st;
  if (!out) return fail(TATTN_E_INVALID, "out is NULL");
  *out = nullptr;
  if (!q || !k || !v) return fail(TATTN_E_INVALID, "q, k and v must be non-NULL");
  if (!aligned16(q) || !aligned16(k) || !aligned16(v)) return fail(TATTN_E_INVALID, "q, k, v must be 16-byte aligned");
  const Layout L = layout_of(*cfg);
  if (!workspace) return fail(TATTN_E_WORKSPACE, "workspace is NULL");
  if (reinterpret_cast<uintptr_t>(workspace) % kAlign) return fail(TATTN_E_WORKSPACE, "workspace must be 256-byte aligned");
  if (workspace_bytes < L.total)
    return fail(TATTN_E_WORKSPACE, "workspace has %zu bytes, %zu needed", workspace_bytes, L.total);
  tattn_plan_s* p = new (std::nothrow) tattn_plan_s;
  if (!p) return fail(TATTN_E_INVALID, "out of host memory");
  st = plan_into(p, cfg, q, k, v, workspace, stream);
  if (st != TATTN_OK) {
    delete p;
    return st;
  }
  *out = p;
  return ok();
}

static tattn_status forward_impl(tattn_plan_t p, const void* q, const void* k, const void* v, void* o,
                                 const int32_t* dslot, int32_t dsteps, uint8_t* dump, void* stream) {
  if (!p) return fail(TATTN_E_INVALID, "plan is NULL");
  if (!q || !o) return fail(TATTN_E_INVALID, "q and o must be non-NULL");
  if (!aligned16(q) || !aligned16(o)) return fail(TATTN_E_INVALID, "q and o must be 16-byte aligned");
  if (k != p->k || v != p->v) return fail(TATTN_E_STATE, "k and v differ from the tensors the plan was built with");
  if (!p->has_tiers) return fail(TATTN_E_STATE, "external-mode plan has no tiers yet (call tattn_plan_set_tiers)");
  AttnArgs a{static_cast<const uint16_t*>(q), static_cast<const uint16_t*>(k), static_cast<const uint16_t*>(v), o,
             p->cfg.out_dtype == TATTN_FP32 ? 1 : 0, p->ws, p->L, p->d, skim_on(p->cfg) ? 1 : 0,
             refine_on(p->cfg) ? 1 : 0, list_cap(p->cfg, p->d), dslot, dump, dsteps};
  hipError_t e = launch_attn(a, static_cast<hipStream_t>(stream));
  if (e != hipSuccess) return hip_fail(e, "attention kernel launch");
  return ok();
}

tattn_status tattn_forward(tattn_plan_t p, const void* q, const void* k, const void* v, void* o, void* stream) {
  return forward_impl(p, q, k, v, o, nullptr, 0, nullptr, stream);
}

tattn_status tattn_forward_dump(tattn_plan_t p, const void* q, const void* k, const void* v, void* o,
                                const int32_t* dump_slot, int32_t dump_steps, uint8_t* dump, void* stream) {
  if (!dump_slot || !dump) return fail(TATTN_E_INVALID, "dump_slot and dump must be non-NULL");
  if (dump_steps < 1) return fail(TATTN_E_INVALID, "dump_steps must be >= 1 (got %d)", dump_steps);
  if (!aligned16(dump)) return fail(TATTN_E_INVALID, "dump must be 16-byte aligned");
  return forward_impl(p, q, k, v, o, dump_slot, dump_steps, dump, stream);
}

tattn_status tattn_attention_static(const tattn_config* cfg, const void* q, const void* k, const void* v, void* o,
                                    void* stream) {
  tattn_status st = validate(cfg);
  if (st != TATTN_OK) return st;
  if (cfg->mode == TATTN_MODE_EXTERNAL)
    return fail(TATTN_E_STATE, "tattn_attention_static routes its own tiers (EXTERNAL mode has none to run)");
  if (!q || !k || !v || !o) return fail(TATTN_E_INVALID, "q, k, v and o must be non-NULL");
  if (!aligned16(q) || !aligned16(k) || !aligned16(v) || !aligned16(o))
    return fail(TATTN_E_INVALID, "q, k, v and o must be 16-byte aligned");
  const size_t need = layout_of(*cfg).total;
  if (need > kStaticScratchBytes)
    return fail(TATTN_E_WORKSPACE, "the problem needs %zu bytes of workspace; the static scratch holds %zu",
                need, (size_t)kStaticScratchBytes);
  void* ws = nullptr;
  st = static_scratch(&ws);
  if (st != TATTN_OK) return st;
  tattn_plan_s p;   // host state on the stack: nothing is allocated
  st = plan_into(&p, cfg, q, k, v, ws, stream);
  if (st != TATTN_OK) return st;
  return forward_impl(&p, q, k, v, o, nullptr, 0, nullptr, stream);
}

tattn_status tattn_list_bound(const tattn_config* cfg, int32_t* bound) {
  tattn_status st = validate(cfg);
  if (st != TATTN_OK) return st;
  if (!bound) return fail(TATTN_E_INVALID, "bound is NULL");
  *bound = list_cap(*cfg, make_dims(*cfg));
  return ok();
}

tattn_status tattn_replan(tattn_plan_t p, const void* q, const void* k, const void* v, void* stream) {
  if (!p) return fail(TATTN_E_INVALID, "plan is NULL");
  if (!q || !k || !v) return fail(TATTN_E_INVALID, "q, k and v must be non-NULL");
  if (!aligned16(q) || !aligned16(k) || !aligned16(v)) return fail(TATTN_E_INVALID, "q, k, v must be 16-byte aligned");
  if (!p->has_tiers) return fail(TATTN_E_STATE, "plan has no tiers yet (nothing to reuse)");
  PoolArgs pa{static_cast<const uint16_t*>(q), static_cast<const uint16_t*>(k), static_cast<const uint16_t*>(v),
              p->ws, p->L, p->d, p->cfg.mode == TATTN_MODE_PRICE ? 1 : 0, skim_on(p->cfg) || refine_on(p->cfg) ? 1 : 0,
              refine_on(p->cfg) ? 1 : 0};
  hipError_t e = launch_pool(pa, static_cast<hipStream_t>(stream));
  if (e != hipSuccess) return hip_fail(e, "pool kernel launch");
  p->k = k;
  p->v = v;
  return ok();
}

static tattn_status copy_out(void* dst, const unsigned char* src, size_t bytes, hipStream_t s) {
  hipError_t e = hipMemcpyAsync(dst, src, bytes, hipMemcpyDeviceToHost, s);
  if (e != hipSuccess) return hip_fail(e, "device-to-host copy");
  return TATTN_OK;
}
static tattn_status sync(hipStream_t s) {
  hipError_t e = hipStreamSynchronize(s);
  if (e != hipSuccess) return hip_fail(e, "stream synchronize");
  return ok();
}

tattn_status tattn_plan_set_tiers(tattn_plan_t p, const uint8_t* host_tiers, void* stream) {
  if (!p) return fail(TATTN_E_INVALID, "plan is NULL");
  if (p->cfg.mode != TATTN_MODE_EXTERNAL) return fail(TATTN_E_STATE, "set_tiers needs a plan built in EXTERNAL mode");
  if (!host_tiers) return fail(TATTN_E_INVALID, "tiers is NULL");
  const size_t n = (size_t)p->d.BH * p->d.Nq * p->d.Nk;
  const unsigned top = skim_on(p->cfg) ? TATTN_SKIM : TATTN_FULL;
  for (size_t i = 0; i < n; i++)
    if (host_tiers[i] > top)
      return fail(TATTN_E_INVALID, "tier byte %u at index %zu is not a tier%s", host_tiers[i], i,
                  host_tiers[i] == TATTN_SKIM ? " (SKIM needs tau_skim > 0)" : "");
  hipStream_t s = static_cast<hipStream_t>(stream);
  hipError_t e = hipMemcpyAsync(p->ws + p->L.tiers, host_tiers, n, hipMemcpyHostToDevice, s);
  if (e != hipSuccess) return hip_fail(e, "host-to-device copy");
  e = launch_compact(router_args(p), s);
  if (e != hipSuccess) return hip_fail(e, "compaction kernel launch");
  tattn_status st = sync(s);
  if (st == TATTN_OK) p->has_tiers = true;
  return st;
}

tattn_status tattn_plan_get_tiers(tattn_plan_t p, uint8_t* host_tiers, float* host_p, void* stream) {
  if (!p) return fail(TATTN_E_INVALID, "plan is NULL");
  if (!p->has_tiers) return fail(TATTN_E_STATE, "plan has no tiers yet");
  hipStream_t s = static_cast<hipStream_t>(stream);
  const size_t n = (size_t)p->d.BH * p->d.Nq * p->d.Nk;
  tattn_status st;
  if (host_tiers && (st = copy_out(host_tiers, p->ws + p->L.tiers, n, s)) != TATTN_OK) return st;
  if (host_p) {
    if (p->cfg.mode == TATTN_MODE_EXTERNAL || p->cfg.mode == TATTN_MODE_ALL_FULL) {
      std::memset(host_p, 0, n * 4);
    } else if ((st = copy_out(host_p, p->ws + p->L.p, n * 4, s)) != TATTN_OK) {
      return st;
    }
  }
  return sync(s);
}

tattn_status tattn_plan_get_lists(tattn_plan_t p, int16_t* host_lists, int32_t* host_counts, void* stream) {
  if (!p) return fail(TATTN_E_INVALID, "plan is NULL");
  if (!p->has_tiers) return fail(TATTN_E_STATE, "plan has no tiers yet");
  hipStream_t s = static_cast<hipStream_t>(stream);
  const size_t rows = (size_t)p->d.BH * p->d.Nq;
  tattn_status st;
  if (host_lists && (st = copy_out(host_lists, p->ws + p->L.lists, rows * p->d.Nk * 2, s)) != TATTN_OK) return st;
  if (host_counts) {
    std::vector<int32_t> c4(rows * 4);
    if ((st = copy_out(c4.data(), p->ws + p->L.counts, rows * 16, s)) != TATTN_OK) return st;
    if ((st = sync(s)) != TATTN_OK) return st;
    for (size_t r = 0; r < rows; r++)
      for (int j = 0; j < 3; j++) host_counts[r * 3 + j] = c4[r * 4 + j];
  }
  return sync(s);
}

tattn_status tattn_plan_get_pool(tattn_plan_t p, float* qbar, float* kbar, float* vbar, float* sq, float* sk, float* sv,
                                 void* stream) {
  if (!p) return fail(TATTN_E_INVALID, "plan is NULL");
  hipStream_t s = static_cast<hipStream_t>(stream);
  const Dims& d = p->d;
  const size_t BH = d.BH;
  tattn_status st;
  if (qbar && (st = copy_out(qbar, p->ws + p->L.qbar, BH * d.Nq * d.D * 4, s)) != TATTN_OK) return st;
  if (kbar && (st = copy_out(kbar, p->ws + p->L.kbar, BH * d.Nk * d.D * 4, s)) != TATTN_OK) return st;
  if (vbar && (st = copy_out(vbar, p->ws + p->L.vbar, BH * d.Nk * d.D * 4, s)) != TATTN_OK) return st;
  if (sq && (st = copy_out(sq, p->ws + p->L.sq, BH * d.Nq * 4, s)) != TATTN_OK) return st;
  if (sk && (st = copy_out(sk, p->ws + p->L.sk, BH * d.Nk * 4, s)) != TATTN_OK) return st;
  if (sv && (st = copy_out(sv, p->ws + p->L.sv, BH * d.Nk * 4, s)) != TATTN_OK) return st;
  return sync(s);
}

tattn_status tattn_plan_get_codes(tattn_plan_t p, uint8_t* host_k8, uint8_t* host_v8, void* stream) {
  if (!p) return fail(TATTN_E_INVALID, "plan is NULL");
  hipStream_t s = static_cast<hipStream_t>(stream);
  const Dims& d = p->d;
  const size_t tile = (size_t)d.Bk * d.D;
  tattn_status st;
  std::vector<uint8_t> slab(p->L.sl.bytes);
  for (size_t bh = 0; bh < (size_t)d.BH; bh++) {
    if ((st = copy_out(slab.data(), p->ws + p->L.slab + bh * p->L.sl.bytes, slab.size(), s)) != TATTN_OK) return st;
    if ((st = sync(s)) != TATTN_OK) return st;
    const uint8_t* k8 = slab.data() + p->L.sl.k8;
    const uint8_t* v8 = slab.data() + p->L.sl.v8t;
    // stored position of key r inside a V^T row of a block
    std::vector<int> vpos(d.Bk);
    for (int e = 0; e < d.Bk; e++) vpos[d.Bk == 64 ? pv8_key(e) : e] = e;
    for (int J = 0; J < d.Nk; J++)
      for (int r = 0; r < d.Bk && J * d.Bk + r < d.N; r++) {
        const size_t n = (size_t)J * d.Bk + r;
        if (host_k8)
          for (int c = 0; c < d.D; c++) host_k8[(bh * d.N + n) * d.D + c] = k8[J * tile + r * d.D + k8_pos(c)];
        if (host_v8)
          for (int c = 0; c < d.D; c++) host_v8[(bh * d.N + n) * d.D + c] = v8[J * tile + c * d.Bk + vpos[r]];
      }
  }
  return ok();
}

// Copy out one MXFP4 region pair of every head's slab in the canonical layout.
static tattn_status get_mx4_pair(tattn_plan_t p, size_t codes_off, size_t scales_off, uint8_t* host_codes,
                                 uint8_t* host_scales, void* stream) {
  hipStream_t s = static_cast<hipStream_t>(stream);
  const Dims& d = p->d;
  const int hb = d.D / 2, nsc = d.D / 32;
  tattn_status st;
  std::vector<uint8_t> slab(p->L.sl.bytes);
  for (size_t bh = 0; bh < (size_t)d.BH; bh++) {
    if ((st = copy_out(slab.data(), p->ws + p->L.slab + bh * p->L.sl.bytes, slab.size(), s)) != TATTN_OK) return st;
    if ((st = sync(s)) != TATTN_OK) return st;
    const uint8_t* k4 = slab.data() + codes_off;
    const uint8_t* k4s = slab.data() + scales_off;
    for (size_t n = 0; n < (size_t)d.N; n++) {   // rows are stored in sequence order
      const size_t at = bh * d.N + n;
      if (host_codes) std::memcpy(host_codes + at * hb, k4 + n * hb, hb);
      if (host_scales) std::memcpy(host_scales + at * nsc, k4s + n * nsc, nsc);
    }
  }
  return ok();
}

tattn_status tattn_plan_get_mx4(tattn_plan_t p, uint8_t* host_k4, uint8_t* host_k4s, void* stream) {
  if (!p) return fail(TATTN_E_INVALID, "plan is NULL");
  if (!skim_on(p->cfg) && !refine_on(p->cfg))
    return fail(TATTN_E_STATE, "MXFP4 copies exist only with the SKIM tier (tau_skim > 0) or low_refine = 1");
  return get_mx4_pair(p, p->L.sl.k4, p->L.sl.k4s, host_k4, host_k4s, stream);
}

tattn_status tattn_plan_get_mx4_residual(tattn_plan_t p, uint8_t* host_k4r, uint8_t* host_k4rs, void* stream) {
  if (!p) return fail(TATTN_E_INVALID, "plan is NULL");
  if (!refine_on(p->cfg)) return fail(TATTN_E_STATE, "the MXFP4 residual exists only with low_refine = 1");
  return get_mx4_pair(p, p->L.sl.k4r, p->L.sl.k4rs, host_k4r, host_k4rs, stream);
}

tattn_status tattn_plan_get_moments(tattn_plan_t p, float* q2, float* m2q, float* kvar, float* m2k, float* vvar,
                                    float* m2v, float* vnorm, void* stream) {
  if (!p) return fail(TATTN_E_INVALID, "plan is NULL");
  if (p->cfg.mode != TATTN_MODE_PRICE) return fail(TATTN_E_STATE, "second moments exist only in PRICE mode");
  hipStream_t s = static_cast<hipStream_t>(stream);
  const Dims& d = p->d;
  const size_t nq = (size_t)d.BH * d.Nq, nk = (size_t)d.BH * d.Nk;
  tattn_status st;
  if (q2 && (st = copy_out(q2, p->ws + p->L.q2, nq * d.D * 4, s)) != TATTN_OK) return st;
  if (m2q && (st = copy_out(m2q, p->ws + p->L.m2q, nq * 4, s)) != TATTN_OK) return st;
  if (kvar && (st = copy_out(kvar, p->ws + p->L.kvar, nk * d.D * 4, s)) != TATTN_OK) return st;
  if (m2k && (st = copy_out(m2k, p->ws + p->L.m2k, nk * 4, s)) != TATTN_OK) return st;
  if (vvar && (st = copy_out(vvar, p->ws + p->L.vvar, nk * 4, s)) != TATTN_OK) return st;
  if (m2v && (st = copy_out(m2v, p->ws + p->L.m2v, nk * 4, s)) != TATTN_OK) return st;
  if (vnorm && (st = copy_out(vnorm, p->ws + p->L.vnorm, nk * 4, s)) != TATTN_OK) return st;
  return sync(s);
}

tattn_status tattn_plan_stats(tattn_plan_t p, tattn_stats* out) {
  if (!p) return fail(TATTN_E_INVALID, "plan is NULL");
  if (!out) return fail(TATTN_E_INVALID, "stats is NULL");
  if (!p->has_tiers) return fail(TATTN_E_STATE, "plan has no tiers yet");
  const Dims& d = p->d;
  std::vector<uint8_t> t((size_t)d.BH * d.Nq * d.Nk);
  hipError_t e = hipDeviceSynchronize();
  if (e != hipSuccess) return hip_fail(e, "device synchronize");
  e = hipMemcpy(t.data(), p->ws + p->L.tiers, t.size(), hipMemcpyDeviceToHost);
  if (e != hipSuccess) return hip_fail(e, "device-to-host copy");
  int32_t flag = 0;
  e = hipMemcpy(&flag, p->ws + p->L.flag, sizeof(flag), hipMemcpyDeviceToHost);
  if (e != hipSuccess) return hip_fail(e, "device-to-host copy");
  if (flag & 1)
    return fail(TATTN_E_STATE, "a forward met a row with more kept tiles than its list bound (%d): the row was cut",
                list_cap(p->cfg, d));
  tattn_stats st{};
  const double D = d.D;
  for (int bh = 0; bh < d.BH; bh++)
    for (int I = 0; I < d.Nq; I++) {
      const double mI = std::min(d.Bq, d.N - I * d.Bq);
      const int r0 = I * d.Bq, r1 = std::min(d.N, (I + 1) * d.Bq);
      const int j0 = r0 / d.Bk, j1 = (r1 - 1) / d.Bk;
      st.n_diag += j1 - j0 + 1;
      const uint8_t* tr = t.data() + ((size_t)bh * d.Nq + I) * d.Nk;
      for (int J = 0; J < d.Nk; J++) {
        const double nJ = std::min(d.Bk, d.N - J * d.Bk);
        if (tr[J] == TATTN_FULL) {
          st.n_full++;
          st.flops_bf16 += 4.0 * mI * nJ * D;
        } else if (tr[J] == TATTN_LOW) {   // fp8 scores (refined: three fp4 passes); fp8 P.V (64-key
          st.n_low++;                      // blocks) or fp16 P.V
          if (refine_on(p->cfg)) st.flops_fp4 += 6.0 * mI * nJ * D;
          else st.flops_fp8 += 2.0 * mI * nJ * D;
          if (d.Bk == 64) st.flops_fp8 += 2.0 * mI * nJ * D;
          else st.flops_bf16 += 2.0 * mI * nJ * D;
        } else if (tr[J] == TATTN_SKIM) {  // fp4 scores; fp8 P.V (64-key blocks) or fp16 P.V
          st.n_skim++;
          st.flops_fp4 += 2.0 * mI * nJ * D;
          if (d.Bk == 64) st.flops_fp8 += 2.0 * mI * nJ * D;
          else st.flops_bf16 += 2.0 * mI * nJ * D;
        } else {
          st.n_skip++;
          st.flops_bf16 += 4.0 * mI * D;
        }
      }
    }
  st.flops_dense = 4.0 * (double)d.N * d.N * D * d.BH;
  *out = st;
  return ok();
}

tattn_status tattn_plan_get_kh(tattn_plan_t p, int32_t* host_kh, double* host_rh) {
  if (!p) return fail(TATTN_E_INVALID, "plan is NULL");
  if (p->cfg.mode != TATTN_MODE_ADAPTIVE) return fail(TATTN_E_STATE, "k_h exists only in ADAPTIVE mode");
  hipError_t e = hipDeviceSynchronize();
  if (e != hipSuccess) return hip_fail(e, "device synchronize");
  if (host_kh && (e = hipMemcpy(host_kh, p->ws + p->L.kh, (size_t)p->d.BH * 4, hipMemcpyDeviceToHost)) != hipSuccess)
    return hip_fail(e, "device-to-host copy");
  if (host_rh && (e = hipMemcpy(host_rh, p->ws + p->L.rh, (size_t)p->d.BH * 8, hipMemcpyDeviceToHost)) != hipSuccess)
    return hip_fail(e, "device-to-host copy");
  return ok();
}

void tattn_plan_destroy(tattn_plan_t p) { delete p; }

const char* tattn_status_str(tattn_status s) {
  switch (s) {
    case TATTN_OK: return "ok";
    case TATTN_E_INVALID: return "invalid argument";
    case TATTN_E_UNSUPPORTED: return "unsupported configuration";
    case TATTN_E_WORKSPACE: return "workspace missing, misaligned or too small";
    case TATTN_E_HIP: return "HIP runtime error";
    case TATTN_E_STATE: return "plan in the wrong state";
  }
  return "unknown status";
}

const char* tattn_last_error(void) { return g_err.c_str(); }

}  // extern "C"
