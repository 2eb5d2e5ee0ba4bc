// C ABI of the DashAttention forward path (include/dash.h): argument checks,
// workspace layout and kernel dispatch.  Every argument visible on the host is
// checked before the first HIP call; nothing here allocates or synchronises.
#include <hip/hip_runtime.h>

#include <cmath>
#include <cstdint>
#include <mutex>

#include "dash.h"
#include "dash_internal.h"

namespace {

using dash::Geom;

constexpr size_t kAlign = 256;

size_t align_up(size_t x) { return (x + kAlign - 1) / kAlign * kAlign; }

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

// Shape checks shared by every entry point.  Fills `g` on success.
dash_status check_shape(const dash_shape* s, int enable_gqa, bool decode, Geom& g) {
  if (!s) return DASH_ERR_INVALID_ARGUMENT;
  if (s->num_seqs < 0 || s->max_seqlen < 0 || s->num_q_heads <= 0 || s->num_kv_heads <= 0 ||
      s->head_dim <= 0 || s->chunk_size <= 0)
    return DASH_ERR_INVALID_ARGUMENT;
  if (s->dtype != DASH_F32 && s->dtype != DASH_BF16) return DASH_ERR_UNSUPPORTED;
  if (s->num_seqs > 65535 || s->num_kv_heads > 65535) return DASH_ERR_UNSUPPORTED;
  if (s->head_dim != 64 && s->head_dim != 128) return DASH_ERR_UNSUPPORTED;
  if (s->chunk_size != 64 && s->chunk_size != 128) return DASH_ERR_UNSUPPORTED;
  if (enable_gqa) {
    if (s->num_q_heads % s->num_kv_heads) return DASH_ERR_INVALID_ARGUMENT;
  } else if (s->num_q_heads != s->num_kv_heads) {
    return DASH_ERR_INVALID_ARGUMENT;
  }
  const int G = s->num_q_heads / s->num_kv_heads;
  if (s->dtype == DASH_BF16) {
    // the group sizes the bf16 kernels are built and tested for
    if (!(G == 1 || G == 2 || G == 4 || G == 8 || G == 16 || G == 32)) return DASH_ERR_UNSUPPORTED;
  }
  const int64_t C_slots = ((int64_t)s->max_seqlen + s->chunk_size - 1) / s->chunk_size;
  if (C_slots > 2048) return DASH_ERR_UNSUPPORTED;
  if (decode) {
    if (s->cu_seqlens) return DASH_ERR_INVALID_ARGUMENT;
    if (s->max_seqlen % s->chunk_size) return DASH_ERR_INVALID_ARGUMENT;
  } else {
    if (s->total_tokens < 0) return DASH_ERR_INVALID_ARGUMENT;
    if (!s->cu_seqlens && s->total_tokens != (int64_t)s->num_seqs * s->max_seqlen)
      return DASH_ERR_INVALID_ARGUMENT;
    if (s->total_tokens > (int64_t)INT32_MAX) return DASH_ERR_UNSUPPORTED;
  }
  g.num_seqs = s->num_seqs;
  g.max_seqlen = s->max_seqlen;
  g.T = decode ? s->num_seqs : s->total_tokens;
  g.cu_seqlens = s->cu_seqlens;
  g.cu_chunks = nullptr;
  g.Hq = s->num_q_heads;
  g.Hkv = s->num_kv_heads;
  g.G = G;
  g.D = s->head_dim;
  g.B = s->chunk_size;
  g.C_slots = (int)C_slots;
  g.W = (int)((C_slots + 63) / 64);
  g.bf16 = (s->dtype == DASH_BF16);
  return DASH_OK;
}

bool finite(float x) { return std::isfinite(x); }

dash_status check_routing(float alpha, float gamma, float sigma, float scale) {
  if (!finite(alpha) || !finite(gamma) || !finite(sigma) || std::isnan(scale))
    return DASH_ERR_INVALID_ARGUMENT;
  if (alpha < 1.f) return DASH_ERR_INVALID_ARGUMENT;
  if (alpha > 2.f) return DASH_ERR_UNSUPPORTED;
  if (gamma <= 0.f || sigma < 0.f) return DASH_ERR_INVALID_ARGUMENT;
  return DASH_OK;
}

float eff_scale(const Geom& g, float scale) {
  return scale > 0.f ? scale : 1.f / std::sqrt((float)g.D);
}

size_t elt(const Geom& g) { return g.bf16 ? 2 : 4; }

// Workspace layouts (offsets in bytes; every piece 256-byte aligned).
// Varlen metadata: cu_chunks then cu_pad, each [num_seqs + 1] int32.
size_t meta_ws(const Geom& g) {
  return g.cu_seqlens ? 2 * align_up(sizeof(int32_t) * (g.num_seqs + 1)) : 0;
}
int32_t* meta_chunks(void* ws) { return reinterpret_cast<int32_t*>(ws); }
int32_t* meta_pad(const Geom& g, void* ws) {
  return reinterpret_cast<int32_t*>(static_cast<char*>(ws) +
                                    align_up(sizeof(int32_t) * (g.num_seqs + 1)));
}
// Row-group flags of the streaming prefill routing (bf16, G = 16 or 32).
size_t flag_bytes(const Geom& g) {
  return (g.bf16 && (g.G == 16 || g.G == 32)) ? align_up((size_t)dash::route_rows_flag_bytes(g))
                                                : 0;
}
// Routing of prefill rows: the streaming kernel (plus its fallback for the
// row groups it flags) where it applies, else one workgroup per row.
hipError_t run_route(const Geom& g, const dash::RouteParams& p, void* flags, hipStream_t s) {
  if (flags && dash::route_rows_supported(g, p)) {
    hipError_t e = dash::launch_route_rows(g, p, static_cast<uint8_t*>(flags), s);
    if (e != hipSuccess) return e;
    return dash::launch_route_fallback(g, p, static_cast<const uint8_t*>(flags), s);
  }
  return dash::launch_route(g, p, s);
}
size_t route_ws(const Geom& g) { return meta_ws(g) + flag_bytes(g); }

size_t vt_bytes(const Geom& g) {
  return dash::prefill_uses_ring(g)
             ? align_up((size_t)g.Hkv * g.D * dash::padded_tokens(g.T, g.num_seqs) * 2)
             : 0;
}

size_t items_bytes(const Geom& g) { return align_up((size_t)dash::prefill_items_capacity(g) * 4); }

struct PrefillWs {
  size_t meta, kbar, mask, logp, vt, kdiag, items, flags, total;
};
PrefillWs prefill_ws(const Geom& g) {
  PrefillWs w{};
  size_t o = 0;
  w.meta = o;
  o += meta_ws(g);
  w.kbar = o;
  o += align_up((size_t)(g.T / g.B) * g.Hkv * g.D * elt(g));
  w.mask = o;
  o += align_up((size_t)g.Hkv * g.T * g.W * 8);
  w.logp = o;
  o += align_up((size_t)g.Hkv * g.T * g.C_slots * 4);
  w.vt = o;
  o += vt_bytes(g);
  w.kdiag = o;  // estimated own-chunk summaries (estimate_diagonal)
  o += align_up((size_t)g.T * g.Hkv * g.D * elt(g));
  w.items = o;  // the attention kernel's varlen work list
  o += items_bytes(g);
  w.flags = o;  // the routing's row-group flags
  o += flag_bytes(g);
  w.total = o;
  return w;
}
struct SparseWs {
  size_t meta, vt, items, total;
};
SparseWs sparse_ws(const Geom& g) {
  SparseWs w{};
  w.meta = 0;
  w.vt = meta_ws(g);
  w.items = w.vt + vt_bytes(g);
  w.total = w.items + items_bytes(g);
  return w;
}
struct DecodeWs {
  size_t mask, logp, acc, ml, ulog, tsx, kdiag, total;
  int nsplit;
};
DecodeWs decode_ws(const Geom& g) {
  DecodeWs w{};
  w.nsplit = dash::decode_num_splits(g);
  size_t o = 0;
  w.mask = o;
  o += align_up((size_t)g.Hkv * g.num_seqs * g.W * 8);
  w.logp = o;
  o += align_up((size_t)g.Hkv * g.num_seqs * g.C_slots * 4);
  w.acc = o;
  o += align_up((size_t)g.num_seqs * g.Hkv * w.nsplit * g.G * g.D * 4);
  w.ml = o;
  o += align_up((size_t)g.num_seqs * g.Hkv * w.nsplit * g.G * 2 * 4);
  w.ulog = o;  // routing logits of the new tokens (bf16 caches)
  if (g.bf16) o += align_up((size_t)g.num_seqs * g.Hkv * g.G * g.C_slots * 4);
  w.tsx = o;   // their per-head thresholds
  if (g.bf16) o += align_up((size_t)g.num_seqs * g.Hkv * g.G * 2 * 4);
  w.kdiag = o;  // the new rows' own-chunk estimates (estimate_diagonal)
  o += align_up((size_t)g.num_seqs * g.Hkv * g.D * elt(g));
  w.total = o;
  return w;
}
// Top-k routing of decode rows (bf16): logits, per-head softmax statistics
// and group scores of the new tokens.
struct RouteDecodeWs {
  size_t ulog, tsx, score, total;
};
RouteDecodeWs route_decode_ws(const Geom& g) {
  RouteDecodeWs w{};
  size_t o = 0;
  w.ulog = o;
  if (g.bf16) o += align_up((size_t)g.num_seqs * g.Hkv * g.G * g.C_slots * 4);
  w.tsx = o;
  if (g.bf16) o += align_up((size_t)g.num_seqs * g.Hkv * g.G * 2 * 4);
  w.score = o;
  if (g.bf16) o += align_up((size_t)g.num_seqs * g.Hkv * g.C_slots * 4);
  w.total = o;
  return w;
}
// Backward of phase 2: D = <dO, O>, and fp32 dQ / dK / dV.
struct BackwardWs {
  size_t meta, delta, dq, dk, dv, total;
};
BackwardWs backward_ws(const Geom& g) {
  BackwardWs w{};
  size_t o = 0;
  w.meta = o;
  o += meta_ws(g);
  w.delta = o;
  o += align_up((size_t)g.Hq * g.T * 4);
  w.dq = o;
  o += align_up((size_t)g.T * g.Hq * g.D * 4);
  w.dk = o;
  o += align_up((size_t)g.T * g.Hkv * g.D * 4);
  w.dv = o;
  o += align_up((size_t)g.T * g.Hkv * g.D * 4);
  w.total = o;
  return w;
}
// Whole prefill backward: the forward's routing recomputed (summaries, mask,
// log-prior, thresholds), the phase-2 backward, the bias gradient and the
// per-head terms of the routing backward.
struct PrefillBwdWs {
  BackwardWs a;
  size_t kbar, mask, logp, tau, db, sc, kbt, dkb, kdiag, dkdiag, flags, rbf, total;
};
PrefillBwdWs prefill_bwd_ws(const Geom& g) {
  PrefillBwdWs w{};
  w.a = backward_ws(g);
  size_t o = w.a.total;
  w.kbar = o;
  o += align_up((size_t)(g.T / g.B) * g.Hkv * g.D * elt(g));
  w.mask = o;
  o += align_up((size_t)g.Hkv * g.T * g.W * 8);
  w.logp = o;
  o += align_up((size_t)g.Hkv * g.T * g.C_slots * 4);
  w.tau = o;
  o += align_up((size_t)g.Hq * g.T * 4);
  w.db = o;
  o += align_up((size_t)g.Hkv * g.T * g.C_slots * 4);
  w.sc = o;
  o += align_up((size_t)g.Hq * g.T * 16);
  w.kbt = o;
  o += align_up((size_t)g.num_seqs * g.Hkv * g.D * dash::route_bwd_cpad(g) * 2);
  w.dkb = o;
  o += align_up((size_t)(g.T / g.B) * g.Hkv * g.D * 4);
  w.kdiag = o;  // estimate_diagonal: the rows' own-chunk estimates and their gradient
  o += align_up((size_t)g.T * g.Hkv * g.D * elt(g));
  w.dkdiag = o;
  o += align_up((size_t)g.T * g.Hkv * g.D * 4);
  w.flags = o;  // the routing's row-group flags (the forward's routing kernels)
  o += flag_bytes(g);
  w.rbf = o;    // the routing backward's rows with more entries than its first pass holds
  o += align_up((size_t)dash::route_flag_stride(g.T) * g.Hkv);
  w.total = o;
  return w;
}
bool backward_supported(const Geom& g) { return g.bf16 && (g.G == 16 || g.G == 32); }
// Decode attention on a given routing: the split partials only.
struct DecodeSparseWs {
  size_t acc, ml, total;
  int nsplit;
};
DecodeSparseWs decode_sparse_ws(const Geom& g) {
  DecodeSparseWs w{};
  w.nsplit = dash::decode_num_splits(g);
  size_t o = 0;
  w.acc = o;
  o += align_up((size_t)g.num_seqs * g.Hkv * w.nsplit * g.G * g.D * 4);
  w.ml = o;
  o += align_up((size_t)g.num_seqs * g.Hkv * w.nsplit * g.G * 2 * 4);
  w.total = o;
  return w;
}
dash_status check_ws(void* ws, size_t have, size_t need) {
  if (have < need) return DASH_ERR_WORKSPACE_TOO_SMALL;
  if (need && !ws) return DASH_ERR_INVALID_ARGUMENT;
  if (need && (reinterpret_cast<uintptr_t>(ws) % kAlign)) return DASH_ERR_INVALID_ARGUMENT;
  return DASH_OK;
}

char* at(void* ws, size_t off) { return static_cast<char*>(ws) + off; }

#define DASH_HIP(call)                              \
  do {                                              \
    if ((call) != hipSuccess) return DASH_ERR_HIP;  \
  } while (0)

// The new tokens a fused decode step appends (dash_attn_decode_append).
struct DecodeAppend {
  const void* k_new = nullptr;
  const void* v_new = nullptr;
  void* k_cache = nullptr;
  void* v_cache = nullptr;
  void* kbar_cache = nullptr;
};

// The decode step on a given workspace (already checked to be large enough).
// app: the step's cache append, or null.  It runs inside the routing's logits
// pass where that pass is the step's first launch (bf16, no own-chunk
// estimates), else as its own launch first.
dash_status decode_run(Geom& g, const DecodeWs& w, const void* q, const void* k_cache,
                       const void* v_cache, const int32_t* seqlens, const void* kbar_cache,
                       const float* qbar, float alpha, float gamma, float sigma,
                       float softmax_scale, int estimate_diagonal, void* out, float* lse,
                       uint64_t* active_blocks, void* workspace, hipStream_t s,
                       const DecodeAppend* app = nullptr) {
  uint64_t* mask = active_blocks ? active_blocks : reinterpret_cast<uint64_t*>(at(workspace, w.mask));
  float* logp = reinterpret_cast<float*>(at(workspace, w.logp));
  dash::RouteParams rp;
  const bool fuse = app && g.bf16 && !estimate_diagonal;
  if (app && !fuse)
    DASH_HIP(dash::launch_cache_append(g, app->k_new, app->v_new, seqlens, qbar, app->k_cache,
                                       app->v_cache, app->kbar_cache, s));
  if (fuse) {
    rp.app_knew = app->k_new;
    rp.app_vnew = app->v_new;
    rp.app_qbar = qbar;
    rp.app_kc = app->k_cache;
    rp.app_vc = app->v_cache;
    rp.app_kbar = app->kbar_cache;
  }
  if (estimate_diagonal) {
    void* kdiag = at(workspace, w.kdiag);
    DASH_HIP(dash::launch_decode_diag(g, k_cache, seqlens, qbar, kdiag, s));
    rp.kdiag = kdiag;
  }
  rp.q = q;
  rp.kbar = kbar_cache;
  rp.alpha = alpha;
  rp.gamma_scale = gamma * eff_scale(g, softmax_scale);
  rp.sigma = sigma;
  rp.mask = mask;
  rp.log_prior = logp;
  rp.seqlens = seqlens;
  rp.rows = g.num_seqs;
  if (g.bf16) {
    rp.ulog = reinterpret_cast<float*>(at(workspace, w.ulog));
    rp.tsx = reinterpret_cast<float*>(at(workspace, w.tsx));
  }
  DASH_HIP(dash::launch_route(g, rp, s));
  dash::DecodeParams dp;
  dp.q = q;
  dp.k = k_cache;
  dp.v = v_cache;
  dp.seqlens = seqlens;
  dp.mask = mask;
  dp.log_prior = logp;
  dp.out = out;
  dp.lse = lse;
  dp.scale = eff_scale(g, softmax_scale);
  dp.part_acc = reinterpret_cast<float*>(at(workspace, w.acc));
  dp.part_ml = reinterpret_cast<float*>(at(workspace, w.ml));
  dp.nsplit = w.nsplit;
  DASH_HIP(dash::launch_decode_attn(g, dp, s));
  return DASH_OK;
}

// Argument checks of a decode step that do not involve the workspace.
dash_status decode_check(const dash_shape* shape, const void* q, const void* k_cache,
                         const void* v_cache, const int32_t* seqlens, const void* kbar_cache,
                         const float* qbar, float alpha, float gamma, float sigma,
                         float softmax_scale, int enable_gqa, int estimate_diagonal,
                         const void* out, Geom& g) {
  dash_status st = check_shape(shape, enable_gqa, true, g);
  if (st != DASH_OK) return st;
  if ((st = check_routing(alpha, gamma, sigma, softmax_scale)) != DASH_OK) return st;
  if (g.num_seqs == 0) return DASH_OK;
  if (!q || !k_cache || !v_cache || !seqlens || !kbar_cache || !out)
    return DASH_ERR_INVALID_ARGUMENT;
  if (estimate_diagonal && !qbar) return DASH_ERR_INVALID_ARGUMENT;
  if (!aligned16(q) || !aligned16(k_cache) || !aligned16(v_cache) || !aligned16(kbar_cache) ||
      !aligned16(out) || !aligned16(qbar))
    return DASH_ERR_INVALID_ARGUMENT;
  if (g.max_seqlen == 0) return DASH_ERR_INVALID_ARGUMENT;
  return DASH_OK;
}

}  // namespace

// ---- the library's own scratch for the allocation-free decode entry point.
// Each GPU that runs the library holds its own copy of this array until the
// process ends.  Host code never passes the array's name to a kernel (on the
// host it is only a stand-in for the symbol): the device address is looked up
// once per device with hipGetSymbolAddress and kept in scratch_dev_ptr.
static __device__ __align__(256) uint8_t scratch[DASH_NOALLOC_SCRATCH_BYTES];

namespace {

constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void* g_scratch_dev_ptr[kMaxDevices] = {};

// Device address of `scratch` on the current device (looked up on the first
// call on that device, under a lock; later calls read the kept pointer).
dash_status scratch_dev_ptr(hipStream_t s, void** out) {
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess) return DASH_ERR_HIP;
  if (s != nullptr) {
    int sdev = -1;
    if (hipStreamGetDevice(s, &sdev) != hipSuccess) return DASH_ERR_HIP;
    if (sdev != dev) return DASH_ERR_INVALID_ARGUMENT;  // the stream's device must be current
  }
  if (dev < 0 || dev >= kMaxDevices) return DASH_ERR_UNSUPPORTED;
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (!g_scratch_dev_ptr[dev]) {
    void* ptr = nullptr;
    if (hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch)) != hipSuccess || !ptr)
      return DASH_ERR_HIP;
    g_scratch_dev_ptr[dev] = ptr;
  }
  *out = g_scratch_dev_ptr[dev];
  return DASH_OK;
}

}  // namespace

extern "C" {

int dash_abi_version(void) { return DASH_ABI_VERSION; }

const char* dash_status_string(dash_status s) {
  switch (s) {
    case DASH_OK: return "ok";
    case DASH_ERR_INVALID_ARGUMENT: return "invalid argument";
    case DASH_ERR_UNSUPPORTED: return "unsupported configuration";
    case DASH_ERR_WORKSPACE_TOO_SMALL: return "workspace too small";
    case DASH_ERR_HIP: return "HIP launch error";
  }
  return "unknown status";
}

dash_status dash_get_layout(const dash_shape* shape, int enable_gqa, dash_layout* out) {
  if (!out) return DASH_ERR_INVALID_ARGUMENT;
  Geom g;
  dash_status st = check_shape(shape, enable_gqa, false, g);
  if (st != DASH_OK) return st;
  out->summary_rows = g.T / g.B;
  out->chunk_slots = g.C_slots;
  out->mask_words = g.W;
  out->group_size = g.G;
  return DASH_OK;
}

size_t dash_workspace_size(int op, const dash_shape* shape) {
  Geom g;
  const bool decode = (op == DASH_OP_DECODE || op == DASH_OP_DECODE_SPARSE ||
                       op == DASH_OP_ROUTE_DECODE);
  if (check_shape(shape, 1, decode, g) != DASH_OK) return 0;
  switch (op) {
    case DASH_OP_SUMMARIZE: return meta_ws(g);
    case DASH_OP_ROUTE: return route_ws(g);
    case DASH_OP_PREFILL: return prefill_ws(g).total;
    case DASH_OP_DECODE: return decode_ws(g).total;
    case DASH_OP_SPARSE: return sparse_ws(g).total;
    case DASH_OP_DECODE_SPARSE: return decode_sparse_ws(g).total;
    case DASH_OP_ROUTE_DECODE: return route_decode_ws(g).total;
    case DASH_OP_BACKWARD: return backward_ws(g).total;
    case DASH_OP_PREFILL_BACKWARD: return prefill_bwd_ws(g).total;
  }
  return 0;
}

dash_status dash_summarize(const dash_shape* shape, const void* k, const float* qbar,
                           void* kbar, void* workspace, size_t workspace_bytes,
                           void* stream) {
  Geom g;
  dash_status st = check_shape(shape, 1, false, g);
  if (st != DASH_OK) return st;
  const size_t need = meta_ws(g);
  if ((st = check_ws(workspace, workspace_bytes, need)) != DASH_OK) return st;
  // nothing to summarise: no pointer is read or written
  if (g.T == 0 || g.num_seqs == 0 || g.T / g.B == 0) return DASH_OK;
  if (!k || !qbar || !kbar) return DASH_ERR_INVALID_ARGUMENT;
  if (!aligned16(k) || !aligned16(qbar) || !aligned16(kbar)) return DASH_ERR_INVALID_ARGUMENT;
  hipStream_t s = static_cast<hipStream_t>(stream);
  if (g.cu_seqlens) {
    g.cu_chunks = meta_chunks(workspace);
    DASH_HIP(dash::launch_varlen_meta(g.cu_seqlens, g.num_seqs, g.B, meta_chunks(workspace),
                                      nullptr, s));
  }
  DASH_HIP(dash::launch_summarize(g, k, qbar, kbar, s));
  return DASH_OK;
}

dash_status dash_summarize_diagonal(const dash_shape* shape, const void* k, const float* qbar,
                                    void* kdiag, void* stream) {
  Geom g;
  dash_status st = check_shape(shape, 1, false, g);
  if (st != DASH_OK) return st;
  if (g.T == 0 || g.num_seqs == 0) return DASH_OK;
  if (!k || !qbar || !kdiag) return DASH_ERR_INVALID_ARGUMENT;
  if (!aligned16(k) || !aligned16(qbar) || !aligned16(kdiag)) return DASH_ERR_INVALID_ARGUMENT;
  DASH_HIP(dash::launch_diag_summary(g, k, qbar, kdiag, static_cast<hipStream_t>(stream)));
  return DASH_OK;
}
dash_status dash_route(const dash_shape* shape, const void* q, const void* kbar,
                       const void* kdiag, float alpha, const float* alpha_per_seq, float gamma,
                       float sigma, float softmax_scale, int enable_gqa,
                       uint64_t* active_blocks, float* log_prior, float* tau, void* workspace,
                       size_t workspace_bytes, void* stream) {
  Geom g;
  dash_status st = check_shape(shape, enable_gqa, false, g);
  if (st != DASH_OK) return st;
  if ((st = check_routing(alpha, gamma, sigma, softmax_scale)) != DASH_OK) return st;
  const size_t need = route_ws(g);
  if ((st = check_ws(workspace, workspace_bytes, need)) != DASH_OK) return st;
  if (g.T == 0 || g.num_seqs == 0) return DASH_OK;
  if (!q || !active_blocks || (!kbar && g.T / g.B > 0)) return DASH_ERR_INVALID_ARGUMENT;
  if (!aligned16(q) || !aligned16(kbar) || !aligned16(kdiag)) return DASH_ERR_INVALID_ARGUMENT;
  hipStream_t s = static_cast<hipStream_t>(stream);
  if (g.cu_seqlens) {
    g.cu_chunks = meta_chunks(workspace);
    DASH_HIP(dash::launch_varlen_meta(g.cu_seqlens, g.num_seqs, g.B, meta_chunks(workspace),
                                      nullptr, s));
  }
  dash::RouteParams p;
  p.q = q;
  p.kbar = kbar;
  p.kdiag = kdiag;
  p.alpha = alpha;
  p.alpha_per_seq = alpha_per_seq;
  p.gamma_scale = gamma * eff_scale(g, softmax_scale);
  p.sigma = sigma;
  p.mask = active_blocks;
  p.log_prior = log_prior;
  p.tau = tau;
  p.rows = g.T;
  DASH_HIP(run_route(g, p, flag_bytes(g) ? at(workspace, meta_ws(g)) : nullptr, s));
  return DASH_OK;
}

dash_status dash_attn_prefill(const dash_shape* shape, const void* q, const void* k,
                              const void* v, const float* qbar, float alpha,
                              const float* alpha_per_seq, float gamma, float sigma,
                              float softmax_scale, int enable_gqa, int estimate_diagonal,
                              void* out, float* lse, uint64_t* active_blocks, void* workspace,
                              size_t workspace_bytes, void* stream) {
  Geom g;
  dash_status st = check_shape(shape, enable_gqa, false, g);
  if (st != DASH_OK) return st;
  if ((st = check_routing(alpha, gamma, sigma, softmax_scale)) != DASH_OK) return st;
  const PrefillWs w = prefill_ws(g);
  if ((st = check_ws(workspace, workspace_bytes, w.total)) != DASH_OK) return st;
  if (g.T == 0 || g.num_seqs == 0) return DASH_OK;  // empty input: nothing is read
  if (!q || !k || !v || !qbar || !out) return DASH_ERR_INVALID_ARGUMENT;
  if (!aligned16(q) || !aligned16(k) || !aligned16(v) || !aligned16(out) || !aligned16(qbar))
    return DASH_ERR_INVALID_ARGUMENT;
  hipStream_t s = static_cast<hipStream_t>(stream);
  if (g.cu_seqlens) {
    void* meta = at(workspace, w.meta);
    g.cu_chunks = meta_chunks(meta);
    g.cu_pad = meta_pad(g, meta);
    DASH_HIP(dash::launch_varlen_meta(g.cu_seqlens, g.num_seqs, g.B, meta_chunks(meta),
                                      meta_pad(g, meta), s));
  }
  void* kbar = at(workspace, w.kbar);
  uint64_t* mask = active_blocks ? active_blocks : reinterpret_cast<uint64_t*>(at(workspace, w.mask));
  float* logp = reinterpret_cast<float*>(at(workspace, w.logp));
  DASH_HIP(dash::launch_summarize(g, k, qbar, kbar, s));
  dash::RouteParams rp;
  if (estimate_diagonal) {
    void* kdiag = at(workspace, w.kdiag);
    DASH_HIP(dash::launch_diag_summary(g, k, qbar, kdiag, s));
    rp.kdiag = kdiag;
  }
  rp.q = q;
  rp.kbar = kbar;
  rp.alpha = alpha;
  rp.alpha_per_seq = alpha_per_seq;
  rp.gamma_scale = gamma * eff_scale(g, softmax_scale);
  rp.sigma = sigma;
  rp.mask = mask;
  rp.log_prior = logp;
  rp.tau = nullptr;
  rp.rows = g.T;
  DASH_HIP(run_route(g, rp, w.flags < w.total ? at(workspace, w.flags) : nullptr, s));
  dash::PrefillParams pp;
  pp.q = q;
  pp.k = k;
  pp.v = v;
  pp.mask = mask;
  pp.log_prior = logp;
  pp.out = out;
  pp.lse = lse;
  pp.scale = eff_scale(g, softmax_scale);
  pp.vt = at(workspace, w.vt);
  pp.Tp = dash::padded_tokens(g.T, g.num_seqs);
  pp.items = reinterpret_cast<uint32_t*>(at(workspace, w.items));
  DASH_HIP(dash::launch_prefill_attn(g, pp, s));
  return DASH_OK;
}

dash_status dash_attn_sparse(const dash_shape* shape, const void* q, const void* k,
                             const void* v, const uint64_t* active_blocks,
                             const float* log_prior, float softmax_scale, int enable_gqa,
                             void* out, float* lse, void* workspace, size_t workspace_bytes,
                             void* stream) {
  Geom g;
  dash_status st = check_shape(shape, enable_gqa, false, g);
  if (st != DASH_OK) return st;
  if (std::isnan(softmax_scale)) return DASH_ERR_INVALID_ARGUMENT;
  const SparseWs w = sparse_ws(g);
  if ((st = check_ws(workspace, workspace_bytes, w.total)) != DASH_OK) return st;
  if (g.T == 0 || g.num_seqs == 0) return DASH_OK;
  if (!q || !k || !v || !active_blocks || !log_prior || !out) return DASH_ERR_INVALID_ARGUMENT;
  if (!aligned16(q) || !aligned16(k) || !aligned16(v) || !aligned16(out))
    return DASH_ERR_INVALID_ARGUMENT;
  hipStream_t s = static_cast<hipStream_t>(stream);
  if (g.cu_seqlens) {
    void* meta = at(workspace, w.meta);
    g.cu_chunks = meta_chunks(meta);
    g.cu_pad = meta_pad(g, meta);
    DASH_HIP(dash::launch_varlen_meta(g.cu_seqlens, g.num_seqs, g.B, meta_chunks(meta),
                                      meta_pad(g, meta), s));
  }
  dash::PrefillParams pp;
  pp.q = q;
  pp.k = k;
  pp.v = v;
  pp.mask = active_blocks;
  pp.log_prior = log_prior;
  pp.out = out;
  pp.lse = lse;
  pp.scale = eff_scale(g, softmax_scale);
  pp.vt = w.items > w.vt ? at(workspace, w.vt) : nullptr;
  pp.Tp = dash::padded_tokens(g.T, g.num_seqs);
  pp.items = w.total > w.items ? reinterpret_cast<uint32_t*>(at(workspace, w.items)) : nullptr;
  DASH_HIP(dash::launch_prefill_attn(g, pp, s));
  return DASH_OK;
}

dash_status dash_attn_decode(const dash_shape* shape, const void* q, const void* k_cache,
                             const void* v_cache, const int32_t* seqlens,
                             const void* kbar_cache, const float* qbar, float alpha,
                             float gamma, float sigma, float softmax_scale, int enable_gqa,
                             int estimate_diagonal, void* out, float* lse,
                             uint64_t* active_blocks, void* workspace,
                             size_t workspace_bytes, void* stream) {
  Geom g;
  dash_status st = decode_check(shape, q, k_cache, v_cache, seqlens, kbar_cache, qbar, alpha,
                                gamma, sigma, softmax_scale, enable_gqa, estimate_diagonal, out,
                                g);
  if (st != DASH_OK) return st;
  const DecodeWs w = decode_ws(g);
  if ((st = check_ws(workspace, workspace_bytes, w.total)) != DASH_OK) return st;
  if (g.num_seqs == 0) return DASH_OK;
  return decode_run(g, w, q, k_cache, v_cache, seqlens, kbar_cache, qbar, alpha, gamma, sigma,
                    softmax_scale, estimate_diagonal, out, lse, active_blocks, workspace,
                    static_cast<hipStream_t>(stream));
}

dash_status dash_attn_decode_append(const dash_shape* shape, const void* q, const void* k_new,
                                    const void* v_new, void* k_cache, void* v_cache,
                                    const int32_t* seqlens, void* kbar_cache, const float* qbar,
                                    float alpha, float gamma, float sigma, float softmax_scale,
                                    int enable_gqa, int estimate_diagonal, void* out, float* lse,
                                    uint64_t* active_blocks, void* workspace,
                                    size_t workspace_bytes, void* stream) {
  Geom g;
  dash_status st = decode_check(shape, q, k_cache, v_cache, seqlens, kbar_cache, qbar, alpha,
                                gamma, sigma, softmax_scale, enable_gqa, estimate_diagonal, out,
                                g);
  if (st != DASH_OK) return st;
  if (g.num_seqs > 0 &&
      (!k_new || !v_new || !qbar || !aligned16(k_new) || !aligned16(v_new)))
    return DASH_ERR_INVALID_ARGUMENT;
  const DecodeWs w = decode_ws(g);
  if ((st = check_ws(workspace, workspace_bytes, w.total)) != DASH_OK) return st;
  if (g.num_seqs == 0) return DASH_OK;
  DecodeAppend app;
  app.k_new = k_new;
  app.v_new = v_new;
  app.k_cache = k_cache;
  app.v_cache = v_cache;
  app.kbar_cache = kbar_cache;
  return decode_run(g, w, q, k_cache, v_cache, seqlens, kbar_cache, qbar, alpha, gamma, sigma,
                    softmax_scale, estimate_diagonal, out, lse, active_blocks, workspace,
                    static_cast<hipStream_t>(stream), &app);
}

dash_status dash_attn_decode_noalloc(const dash_shape* shape, const void* q,
                                     const void* k_cache, const void* v_cache,
                                     const int32_t* seqlens, const void* kbar_cache,
                                     const float* qbar, float alpha, float gamma, float sigma,
                                     float softmax_scale, int enable_gqa,
                                     int estimate_diagonal, void* out, float* lse,
                                     uint64_t* active_blocks, void* stream) {
  Geom g;
  dash_status st = decode_check(shape, q, k_cache, v_cache, seqlens, kbar_cache, qbar, alpha,
                                gamma, sigma, softmax_scale, enable_gqa, estimate_diagonal, out,
                                g);
  if (st != DASH_OK) return st;
  const DecodeWs w = decode_ws(g);
  if (w.total > (size_t)DASH_NOALLOC_SCRATCH_BYTES) return DASH_ERR_UNSUPPORTED;
  if (g.num_seqs == 0) return DASH_OK;
  hipStream_t s = static_cast<hipStream_t>(stream);
  void* ws = nullptr;
  if ((st = scratch_dev_ptr(s, &ws)) != DASH_OK) return st;
  return decode_run(g, w, q, k_cache, v_cache, seqlens, kbar_cache, qbar, alpha, gamma, sigma,
                    softmax_scale, estimate_diagonal, out, lse, active_blocks, ws, s);
}

dash_status dash_prefill_schedule(const dash_shape* shape, int enable_gqa, uint32_t* items,
                                  size_t capacity, int* positions_per_tile, void* stream) {
  Geom g;
  dash_status st = check_shape(shape, enable_gqa, false, g);
  if (st != DASH_OK) return st;
  if (!positions_per_tile) return DASH_ERR_INVALID_ARGUMENT;
  const int64_t cap = dash::prefill_items_capacity(g);
  if (cap <= 0) return DASH_ERR_UNSUPPORTED;
  if (capacity < (size_t)cap) return DASH_ERR_WORKSPACE_TOO_SMALL;
  if (!items) return DASH_ERR_INVALID_ARGUMENT;
  const int P = dash::prefill_positions_per_tile(g);
  *positions_per_tile = P;
  DASH_HIP(dash::launch_prefill_schedule(g, P, items, cap, static_cast<hipStream_t>(stream)));
  return DASH_OK;
}

dash_status dash_probe_peak(int kind, const void* src, size_t bytes, int iters, void* sink,
                           size_t sink_bytes, double* work, void* stream) {
  if (!work || !sink || sink_bytes < 1024 || !aligned16(sink)) return DASH_ERR_INVALID_ARGUMENT;
  if (kind == 0) {
    if (iters <= 0) return DASH_ERR_INVALID_ARGUMENT;
  } else if (kind == 1) {
    if (!src || !aligned16(src) || bytes < 16) return DASH_ERR_INVALID_ARGUMENT;
  } else {
    return DASH_ERR_INVALID_ARGUMENT;
  }
  DASH_HIP(dash::launch_probe(kind, src, bytes, iters, sink, work,
                              static_cast<hipStream_t>(stream)));
  return DASH_OK;
}

size_t dash_noalloc_scratch_need(const dash_shape* shape) {
  Geom g;
  if (check_shape(shape, 1, true, g) != DASH_OK) return 0;
  return decode_ws(g).total;
}

dash_status dash_route_topk(const dash_shape* shape, const void* q, const void* kbar,
                            int topk, float gamma, float softmax_scale, int enable_gqa,
                            const int32_t* decode_seqlens, uint64_t* active_blocks,
                            float* log_prior, void* workspace, size_t workspace_bytes,
                            void* stream) {
  const bool decode = decode_seqlens != nullptr;
  Geom g;
  dash_status st = check_shape(shape, enable_gqa, decode, g);
  if (st != DASH_OK) return st;
  if ((st = check_routing(1.f, gamma, 0.f, softmax_scale)) != DASH_OK) return st;
  if (topk <= 0) return DASH_ERR_INVALID_ARGUMENT;
  const RouteDecodeWs dw = route_decode_ws(g);
  const size_t need = decode ? dw.total : meta_ws(g);
  if ((st = check_ws(workspace, workspace_bytes, need)) != DASH_OK) return st;
  if (g.T == 0 || g.num_seqs == 0) return DASH_OK;
  const bool any_summary = decode ? g.max_seqlen >= g.B : g.T / g.B > 0;
  if (!q || !active_blocks || (!kbar && any_summary)) return DASH_ERR_INVALID_ARGUMENT;
  if (!aligned16(q) || !aligned16(kbar)) return DASH_ERR_INVALID_ARGUMENT;
  if (decode && g.max_seqlen == 0) return DASH_ERR_INVALID_ARGUMENT;
  hipStream_t s = static_cast<hipStream_t>(stream);
  if (!decode && g.cu_seqlens) {
    g.cu_chunks = meta_chunks(workspace);
    DASH_HIP(dash::launch_varlen_meta(g.cu_seqlens, g.num_seqs, g.B, meta_chunks(workspace),
                                      nullptr, s));
  }
  dash::RouteParams p;
  p.q = q;
  p.kbar = kbar;
  p.alpha = 1.f;
  p.gamma_scale = gamma * eff_scale(g, softmax_scale);
  p.sigma = 0.f;
  p.mask = active_blocks;
  p.log_prior = log_prior;
  p.seqlens = decode_seqlens;
  p.rows = g.T;
  p.topk = topk;
  if (decode && g.bf16) {
    p.ulog = reinterpret_cast<float*>(at(workspace, dw.ulog));
    p.tsx = reinterpret_cast<float*>(at(workspace, dw.tsx));
    p.score = reinterpret_cast<float*>(at(workspace, dw.score));
  }
  DASH_HIP(dash::launch_route(g, p, s));
  return DASH_OK;
}

dash_status dash_cache_append(const dash_shape* shape, const void* k_new, const void* v_new,
                              const int32_t* seqlens, const float* qbar, void* k_cache,
                              void* v_cache, void* kbar_cache, void* stream) {
  Geom g;
  dash_status st = check_shape(shape, 1, true, g);
  if (st != DASH_OK) return st;
  if (g.num_seqs == 0) return DASH_OK;
  if (!k_new || !v_new || !seqlens || !qbar || !k_cache || !v_cache || !kbar_cache)
    return DASH_ERR_INVALID_ARGUMENT;
  if (!aligned16(k_new) || !aligned16(v_new) || !aligned16(k_cache) || !aligned16(v_cache) ||
      !aligned16(kbar_cache) || !aligned16(qbar))
    return DASH_ERR_INVALID_ARGUMENT;
  if (g.max_seqlen == 0) return DASH_ERR_INVALID_ARGUMENT;
  DASH_HIP(dash::launch_cache_append(g, k_new, v_new, seqlens, qbar, k_cache, v_cache,
                                     kbar_cache, static_cast<hipStream_t>(stream)));
  return DASH_OK;
}

dash_status dash_attn_sparse_backward(const dash_shape* shape, const void* q, const void* k,
                                      const void* v, const void* out, const void* dout,
                                      const float* lse, const uint64_t* active_blocks,
                                      const float* log_prior, float softmax_scale,
                                      int enable_gqa, void* dq, void* dk, void* dv,
                                      float* dbias, void* workspace, size_t workspace_bytes,
                                      void* stream) {
  Geom g;
  dash_status st = check_shape(shape, enable_gqa, false, g);
  if (st != DASH_OK) return st;
  if (std::isnan(softmax_scale)) return DASH_ERR_INVALID_ARGUMENT;
  if (g.T > 0 && !backward_supported(g)) return DASH_ERR_UNSUPPORTED;
  const BackwardWs w = backward_ws(g);
  if ((st = check_ws(workspace, workspace_bytes, w.total)) != DASH_OK) return st;
  if (g.T == 0 || g.num_seqs == 0) return DASH_OK;
  if (!q || !k || !v || !out || !dout || !lse || !active_blocks || !log_prior || !dq || !dk ||
      !dv || !dbias)
    return DASH_ERR_INVALID_ARGUMENT;
  if (!aligned16(q) || !aligned16(k) || !aligned16(v) || !aligned16(out) || !aligned16(dout) ||
      !aligned16(dq) || !aligned16(dk) || !aligned16(dv) || !aligned16(dbias))
    return DASH_ERR_INVALID_ARGUMENT;
  hipStream_t s = static_cast<hipStream_t>(stream);
  if (g.cu_seqlens) {
    void* meta = at(workspace, w.meta);
    g.cu_chunks = meta_chunks(meta);
    g.cu_pad = meta_pad(g, meta);
    DASH_HIP(dash::launch_varlen_meta(g.cu_seqlens, g.num_seqs, g.B, meta_chunks(meta),
                                      meta_pad(g, meta), s));
  }
  dash::BwdParams p;
  p.q = q;
  p.k = k;
  p.v = v;
  p.dout = dout;
  p.lse = lse;
  p.delta = reinterpret_cast<float*>(at(workspace, w.delta));
  p.mask = active_blocks;
  p.log_prior = log_prior;
  p.scale = eff_scale(g, softmax_scale);
  p.dq = reinterpret_cast<float*>(at(workspace, w.dq));
  p.dbias = dbias;
  float* dkw = reinterpret_cast<float*>(at(workspace, w.dk));
  float* dvw = reinterpret_cast<float*>(at(workspace, w.dv));
  DASH_HIP(dash::launch_bwd_delta(g, out, dout, reinterpret_cast<float*>(at(workspace, w.delta)), s));
  DASH_HIP(dash::launch_zero(dbias, (int64_t)g.Hkv * g.T * g.C_slots, s));
  DASH_HIP(dash::launch_bwd_dq(g, p, s));
  DASH_HIP(dash::launch_bwd_dkdv(g, p, dkw, dvw, s));
  DASH_HIP(dash::launch_to_bf16(p.dq, dq, g.T * g.Hq * g.D, s));
  DASH_HIP(dash::launch_to_bf16(dkw, dk, g.T * g.Hkv * g.D, s));
  DASH_HIP(dash::launch_to_bf16(dvw, dv, g.T * g.Hkv * g.D, s));
  return DASH_OK;
}

dash_status dash_attn_prefill_backward(const dash_shape* shape, const void* q, const void* k,
                                       const void* v, const float* qbar, float alpha,
                                       const float* alpha_per_seq, float gamma, float sigma,
                                       float softmax_scale, int enable_gqa,
                                       int estimate_diagonal, const void* out, const void* dout,
                                       const float* lse, void* dq, void* dk, void* dv,
                                       float* dqbar, void* workspace, size_t workspace_bytes,
                                       void* stream) {
  Geom g;
  dash_status st = check_shape(shape, enable_gqa, false, g);
  if (st != DASH_OK) return st;
  if ((st = check_routing(alpha, gamma, sigma, softmax_scale)) != DASH_OK) return st;
  if (g.T > 0 && !backward_supported(g)) return DASH_ERR_UNSUPPORTED;
  const PrefillBwdWs w = prefill_bwd_ws(g);
  if ((st = check_ws(workspace, workspace_bytes, w.total)) != DASH_OK) return st;
  if (g.T == 0 || g.num_seqs == 0) return DASH_OK;
  if (!q || !k || !v || !qbar || !out || !dout || !lse || !dq || !dk || !dv || !dqbar)
    return DASH_ERR_INVALID_ARGUMENT;
  if (!aligned16(q) || !aligned16(k) || !aligned16(v) || !aligned16(qbar) || !aligned16(out) ||
      !aligned16(dout) || !aligned16(dq) || !aligned16(dk) || !aligned16(dv) ||
      !aligned16(dqbar))
    return DASH_ERR_INVALID_ARGUMENT;
  hipStream_t s = static_cast<hipStream_t>(stream);
  if (g.cu_seqlens) {
    void* meta = at(workspace, w.a.meta);
    g.cu_chunks = meta_chunks(meta);
    g.cu_pad = meta_pad(g, meta);
    DASH_HIP(dash::launch_varlen_meta(g.cu_seqlens, g.num_seqs, g.B, meta_chunks(meta),
                                      meta_pad(g, meta), s));
  }
  // the forward's routing, recomputed by the same kernels
  void* kbar = at(workspace, w.kbar);
  uint64_t* mask = reinterpret_cast<uint64_t*>(at(workspace, w.mask));
  float* logp = reinterpret_cast<float*>(at(workspace, w.logp));
  float* tau = reinterpret_cast<float*>(at(workspace, w.tau));
  DASH_HIP(dash::launch_summarize(g, k, qbar, kbar, s));
  dash::RouteParams rp;
  void* kdiag = nullptr;
  if (estimate_diagonal) {
    kdiag = at(workspace, w.kdiag);
    DASH_HIP(dash::launch_diag_summary(g, k, qbar, kdiag, s));
    rp.kdiag = kdiag;
  }
  rp.q = q;
  rp.kbar = kbar;
  rp.alpha = alpha;
  rp.alpha_per_seq = alpha_per_seq;
  rp.gamma_scale = gamma * eff_scale(g, softmax_scale);
  rp.sigma = sigma;
  rp.mask = mask;
  rp.log_prior = logp;
  rp.tau = tau;
  rp.rows = g.T;
  DASH_HIP(run_route(g, rp, w.flags < w.total ? at(workspace, w.flags) : nullptr, s));
  // phase 2
  dash::BwdParams p;
  p.q = q;
  p.k = k;
  p.v = v;
  p.dout = dout;
  p.lse = lse;
  p.delta = reinterpret_cast<float*>(at(workspace, w.a.delta));
  p.mask = mask;
  p.log_prior = logp;
  p.scale = eff_scale(g, softmax_scale);
  p.dq = reinterpret_cast<float*>(at(workspace, w.a.dq));
  p.dbias = reinterpret_cast<float*>(at(workspace, w.db));
  float* dkw = reinterpret_cast<float*>(at(workspace, w.a.dk));
  float* dvw = reinterpret_cast<float*>(at(workspace, w.a.dv));
  DASH_HIP(dash::launch_bwd_delta(g, out, dout, reinterpret_cast<float*>(at(workspace, w.a.delta)), s));
  DASH_HIP(dash::launch_zero(p.dbias, (int64_t)g.Hkv * g.T * g.C_slots, s));
  DASH_HIP(dash::launch_bwd_dq(g, p, s));
  DASH_HIP(dash::launch_bwd_dkdv(g, p, dkw, dvw, s));
  // phases 1 and 0
  dash::RouteBwdParams rb;
  rb.q = q;
  rb.kbar = kbar;
  rb.k = k;
  rb.qbar = qbar;
  rb.tau = tau;
  rb.mask = reinterpret_cast<const unsigned long long*>(mask);
  rb.db = p.dbias;
  rb.sc = reinterpret_cast<float4*>(at(workspace, w.sc));
  rb.dq = p.dq;
  rb.dk = dkw;
  rb.dqbar = dqbar;
  rb.alpha = alpha;
  rb.alpha_per_seq = alpha_per_seq;
  rb.gamma_scale = rp.gamma_scale;
  rb.sigma = sigma;
  rb.kbt = reinterpret_cast<const uint16_t*>(at(workspace, w.kbt));
  rb.dkb = reinterpret_cast<float*>(at(workspace, w.dkb));
  rb.cpad = dash::route_bwd_cpad(g);
  rb.rflags = reinterpret_cast<uint8_t*>(at(workspace, w.rbf));
  rb.kdiag = kdiag;
  rb.dkdiag = reinterpret_cast<float*>(at(workspace, w.dkdiag));
  DASH_HIP(dash::launch_zero(dqbar, (int64_t)g.Hkv * g.D, s));
  DASH_HIP(dash::launch_zero(rb.dkb, (int64_t)(g.T / g.B) * g.Hkv * g.D, s));
  DASH_HIP(dash::launch_route_bwd(g, rb, s));
  DASH_HIP(dash::launch_to_bf16(p.dq, dq, g.T * g.Hq * g.D, s));
  DASH_HIP(dash::launch_to_bf16(dkw, dk, g.T * g.Hkv * g.D, s));
  DASH_HIP(dash::launch_to_bf16(dvw, dv, g.T * g.Hkv * g.D, s));
  return DASH_OK;
}

dash_status dash_attn_decode_sparse(const dash_shape* shape, const void* q,
                                    const void* k_cache, const void* v_cache,
                                    const int32_t* seqlens, const uint64_t* active_blocks,
                                    const float* log_prior, float softmax_scale,
                                    int enable_gqa, void* out, float* lse, void* workspace,
                                    size_t workspace_bytes, void* stream) {
  Geom g;
  dash_status st = check_shape(shape, enable_gqa, true, g);
  if (st != DASH_OK) return st;
  if (std::isnan(softmax_scale)) return DASH_ERR_INVALID_ARGUMENT;
  const DecodeSparseWs w = decode_sparse_ws(g);
  if ((st = check_ws(workspace, workspace_bytes, w.total)) != DASH_OK) return st;
  if (g.num_seqs == 0) return DASH_OK;
  if (!q || !k_cache || !v_cache || !seqlens || !active_blocks || !log_prior || !out)
    return DASH_ERR_INVALID_ARGUMENT;
  if (!aligned16(q) || !aligned16(k_cache) || !aligned16(v_cache) || !aligned16(out))
    return DASH_ERR_INVALID_ARGUMENT;
  if (g.max_seqlen == 0) return DASH_ERR_INVALID_ARGUMENT;
  hipStream_t s = static_cast<hipStream_t>(stream);
  dash::DecodeParams dp;
  dp.q = q;
  dp.k = k_cache;
  dp.v = v_cache;
  dp.seqlens = seqlens;
  dp.mask = active_blocks;
  dp.log_prior = log_prior;
  dp.out = out;
  dp.lse = lse;
  dp.scale = eff_scale(g, softmax_scale);
  dp.part_acc = reinterpret_cast<float*>(at(workspace, w.acc));
  dp.part_ml = reinterpret_cast<float*>(at(workspace, w.ml));
  dp.nsplit = w.nsplit;
  DASH_HIP(dash::launch_decode_attn(g, dp, s));
  return DASH_OK;
}

}  // extern "C"
