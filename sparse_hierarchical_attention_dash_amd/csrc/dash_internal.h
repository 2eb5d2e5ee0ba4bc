// Internal launch interface between the C ABI (dash_api.cpp) and the kernels.
// Everything here has been validated on the host before it is called.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace dash {

// Geometry of one call, validated and derived on the host.
struct Geom {
  int num_seqs = 0;
  int max_seqlen = 0;
  int64_t T = 0;                        // packed token rows (prefill / route)
  const int32_t* cu_seqlens = nullptr;  // device [num_seqs+1] or null
  const int32_t* cu_chunks = nullptr;   // device [num_seqs+1] (workspace) or null
  const int32_t* cu_pad = nullptr;      // device [num_seqs+1]: 64-padded token offsets, or null
  int Hq = 0, Hkv = 0, G = 0, D = 0, B = 0;
  int C_slots = 0;                      // ceil(max_seqlen / B)
  int W = 0;                            // ceil(C_slots / 64)
  bool bf16 = true;
};

// a0: cu_chunks[s] = sum_{s' < s} floor(L_s' / B) and, when cu_pad is not
// null, cu_pad[s] = sum_{s' < s} 64 * ceil(L_s' / 64).
hipError_t launch_varlen_meta(const int32_t* cu_seqlens, int num_seqs, int B,
                              int32_t* cu_chunks, int32_t* cu_pad, hipStream_t st);

// Columns of a sequence's keys in the 64-padded V^T layout.
inline int64_t padded_tokens(int64_t T, int num_seqs) { return T + 64ll * num_seqs; }

// K0: chunk summaries.
hipError_t launch_summarize(const Geom& g, const void* k, const float* qbar,
                            void* kbar, hipStream_t st);

// Estimated summary of each position's own partial chunk (the learned-query
// attention over its chunk's keys up to the position): prefill, every token
// row, kdiag [T, Hkv, D]; decode, the new row of each batch entry from its
// cache, kdiag [batch, Hkv, D].
hipError_t launch_diag_summary(const Geom& g, const void* k, const float* qbar, void* kdiag,
                               hipStream_t st);
hipError_t launch_decode_diag(const Geom& g, const void* k_cache, const int32_t* seqlens,
                              const float* qbar, void* kdiag, hipStream_t st);

// measurement probes (probe.hip): kind 0 = MFMA issue loop, 1 = HBM read stream;
// *work receives the FLOPs (0) or bytes (1) one launch processes
hipError_t launch_probe(int kind, const void* src, size_t bytes, int iters, void* sink,
                        double* work, hipStream_t st);

// Decode-cache upkeep: append the new tokens' K/V rows (position seqlens[b]-1
// of caches [batch, cap, Hkv, D]) and summarise each chunk they complete.
hipError_t launch_cache_append(const Geom& g, const void* k_new, const void* v_new,
                               const int32_t* seqlens, const float* qbar, void* k_cache,
                               void* v_cache, void* kbar_cache, hipStream_t st);

// K1: routing.  Prefill mode routes every packed token row; decode mode
// (seqlens != null) routes batch entry b at position seqlens[b] - 1 against
// summary rows b * (max_seqlen / B) ...
struct RouteParams {
  const void* q = nullptr;
  const void* kbar = nullptr;
  float alpha = 1.5f;
  const float* alpha_per_seq = nullptr;
  float gamma_scale = 1.f;              // gamma * s
  float sigma = 1.f;
  uint64_t* mask = nullptr;             // [Hkv, rows, W]
  float* log_prior = nullptr;           // [Hkv, rows, C_slots] or null
  float* tau = nullptr;                 // [Hq, rows] or null
  const int32_t* seqlens = nullptr;     // decode mode when non-null
  int64_t rows = 0;                     // T (prefill) or batch (decode)
  float* ulog = nullptr;                // decode, bf16: logits scratch [rows, Hkv, G, C_slots]
  float* tsx = nullptr;                 // decode, bf16: per-head threshold scratch [rows, Hkv, G, 2]
  int topk = 0;                         // > 0: top-k routing (group softmax scores, bias 0)
  float* score = nullptr;               // decode, bf16, top-k: group scores scratch [rows, Hkv, C_slots]
  const void* kdiag = nullptr;          // [rows, Hkv, D] estimated own-chunk summaries, or null:
                                        // one more entmax entry per row (after the routed chunks)
  int64_t row0 = 0;                     // first row of the launch (prefill row ranges)
  // decode, bf16, no own-chunk estimates: the append of the step's new tokens
  // (append_token), run by one more column of the logits pass's workgroups,
  // or null.  The logits never read what it writes: a query routes only the
  // chunks before its own, and the append completes at most the query's own.
  const void* app_knew = nullptr;       // [rows, Hkv, D]
  const void* app_vnew = nullptr;
  const float* app_qbar = nullptr;      // [Hkv, D]
  void* app_kc = nullptr;               // caches [rows, cap, Hkv, D] (written)
  void* app_vc = nullptr;
  void* app_kbar = nullptr;             // [rows, cap / B, Hkv, D] (written)
};
hipError_t launch_route(const Geom& g, const RouteParams& p, hipStream_t st);
// Streaming routing of prefill rows (route_rows.hip) where it applies (bf16,
// G = 16 or 32, entmax, no own-chunk estimates, all rows of the call), with
// route_fallback_kernel for the row groups it flags.  flags: workspace of
// route_rows_flag_bytes(g) bytes (no initial contents needed).
bool route_rows_supported(const Geom& g, const RouteParams& p);
// Bytes between two KV heads' flag rows (flags[h * stride + row], 0 or 1):
// whole 16-byte words, so that the fallback reads them four rows at a time.
__host__ __device__ inline int64_t route_flag_stride(int64_t rows) { return (rows + 15) & ~(int64_t)15; }
int route_rows_per_group(const Geom& g);
int64_t route_rows_flag_bytes(const Geom& g);
hipError_t launch_route_rows(const Geom& g, const RouteParams& p, uint8_t* flags,
                             hipStream_t st);
hipError_t launch_route_fallback(const Geom& g, const RouteParams& p, const uint8_t* flags,
                                 hipStream_t st);

// K2p: prefill attention over the active chunks and the diagonal.
struct PrefillParams {
  void* vt = nullptr;                   // workspace V^T [Hkv, D, Tp] (bf16, G >= 16)
  int64_t Tp = 0;                       // padded columns of vt
  const void* q = nullptr;
  const void* k = nullptr;
  const void* v = nullptr;
  const uint64_t* mask = nullptr;       // [Hkv, T, W]
  const float* log_prior = nullptr;     // [Hkv, T, C_slots]
  void* out = nullptr;
  float* lse = nullptr;                 // [Hq, T] or null
  float scale = 0.f;
  uint32_t* items = nullptr;            // workspace: varlen work list (prefill_items_capacity)
};
hipError_t launch_prefill_attn(const Geom& g, const PrefillParams& p, hipStream_t st);
// Entries of the varlen work list of the G >= 16 prefill kernels (0 when the
// call does not use one): ceil(T / 8) + num_seqs, enough for P >= 8.
int64_t prefill_items_capacity(const Geom& g);
// Positions per workgroup tile of the G >= 16 prefill attention kernel.
int prefill_positions_per_tile(const Geom& g);
// The longest-first work list of a varlen pack with P positions per tile
// (entries (sequence << 16) | tile, 0xffffffff past the end), cap entries.
hipError_t launch_prefill_schedule(const Geom& g, int P, uint32_t* items, int64_t cap,
                                   hipStream_t st);
// True when launch_prefill_attn runs the V^T + LDS-ring path (needs p.vt).
bool prefill_uses_ring(const Geom& g);

// Backward of phase 2 for a given routing (bf16, G >= 16).
struct BwdParams {
  const void* q = nullptr;              // [T, Hq, D]
  const void* k = nullptr;              // [T, Hkv, D]
  const void* v = nullptr;
  const void* dout = nullptr;           // [T, Hq, D]
  const float* lse = nullptr;           // [Hq, T] natural log, from the forward
  const float* delta = nullptr;         // [Hq, T] <dO, O>
  const uint64_t* mask = nullptr;       // [Hkv, T, W]
  const float* log_prior = nullptr;     // [Hkv, T, C_slots]
  float scale = 0.f;
  float* dq = nullptr;                  // [T, Hq, D] fp32 (written)
  float* dbias = nullptr;               // [Hkv, T, C_slots] fp32 (accumulated; zeroed first)
};
hipError_t launch_bwd_dq(const Geom& g, const BwdParams& p, hipStream_t st);
hipError_t launch_bwd_delta(const Geom& g, const void* out, const void* dout, float* delta,
                            hipStream_t st);
hipError_t launch_bwd_dkdv(const Geom& g, const BwdParams& p, float* dk, float* dv,
                           hipStream_t st);
hipError_t launch_to_bf16(const float* src, void* dst, int64_t n, hipStream_t st);
hipError_t launch_zero(float* x, int64_t n, hipStream_t st);

// Backward of phases 1 and 0 (bf16, G = 16 or 32).
struct RouteBwdParams {
  const void* q = nullptr;              // [T, Hq, D]
  const void* kbar = nullptr;           // [T/B rows, Hkv, D]
  const void* k = nullptr;              // [T, Hkv, D]
  const float* qbar = nullptr;          // [Hkv, D]
  const float* tau = nullptr;           // [Hq, T] the forward's thresholds (u units)
  const unsigned long long* mask = nullptr;  // [Hkv, T, W]
  float* db = nullptr;                  // [Hkv, T, C_slots] bias gradient in, dp out
  float4* sc = nullptr;                 // [Hq, T] per head: threshold or max, softmax sum, rho
  float* dq = nullptr;                  // [T, Hq, D] fp32, accumulated
  float* dk = nullptr;                  // [T, Hkv, D] fp32, accumulated
  float* dqbar = nullptr;               // [Hkv, D] fp32, accumulated (zeroed first)
  const uint16_t* kbt = nullptr;        // [seqs, Hkv, D, cpad] bf16 (filled here)
  const void* kdiag = nullptr;          // [T, Hkv, D] own-chunk estimates, or null
  float* dkdiag = nullptr;              // [T, Hkv, D] fp32, their gradient (written)
  float* dkb = nullptr;                 // [T/B rows, Hkv, D] fp32 dk_bar (zeroed first)
  int cpad = 0;                         // route_bwd_cpad(g)
  uint8_t* rflags = nullptr;            // [Hkv, route_flag_stride(T)]: rows left to the wide pass
  float alpha = 1.5f;
  const float* alpha_per_seq = nullptr; // [num_seqs] or null (varlen)
  float gamma_scale = 1.f;              // gamma * s
  float sigma = 1.f;
};
int route_bwd_cpad(const Geom& g);  // complete chunks per sequence, rounded up to 32
hipError_t launch_route_bwd(const Geom& g, const RouteBwdParams& p, hipStream_t st);
hipError_t launch_vt_transpose(const Geom& g, const void* src, void* dst, int64_t Tp,
                               hipStream_t st);

// K2d + K4: split-K decode attention and the combine of the partials.
struct DecodeParams {
  const void* q = nullptr;              // [batch, Hq, D]
  const void* k = nullptr;              // [batch, cap, Hkv, D]
  const void* v = nullptr;
  const int32_t* seqlens = nullptr;     // [batch]
  const uint64_t* mask = nullptr;       // [Hkv, batch, W]
  const float* log_prior = nullptr;     // [Hkv, batch, C_slots]
  void* out = nullptr;                  // [batch, Hq, D]
  float* lse = nullptr;                 // [Hq, batch] or null
  float scale = 0.f;
  float* part_acc = nullptr;            // [batch, Hkv, nsplit, G, D]
  float* part_ml = nullptr;             // [batch, Hkv, nsplit, G, 2]
  int nsplit = 1;
};
int decode_num_splits(const Geom& g);
hipError_t launch_decode_attn(const Geom& g, const DecodeParams& p, hipStream_t st);

}  // namespace dash
