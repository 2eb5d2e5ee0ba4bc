// Phase 0: learned-query chunk summaries ("Fase 0: Lokale Chunk Samenvatting"
// of the gist.science technical summary), plus the varlen chunk offsets.
//
// k_bar[c,h] = sum_t softmax_t(<q_bar[h], k[cB+t,h]> / sqrt(D)) k[cB+t,h]
//
// One wave per (chunk, KV head).  The chunk's B keys are streamed once from
// HBM with 16-byte loads; lane groups of D/8 (bf16) or D/4 (fp32) lanes cover
// one key row, so each load instruction reads whole rows contiguously.  Each
// lane group keeps a running (max, sum, weighted key) over its keys (online
// softmax), and the groups are merged with cross-lane shuffles at the end.
// The result is rounded to the storage dtype once.  HBM-bound: it reads K once.
#include "chunk_summary.h"
#include "dash_device.h"
#include "dash_internal.h"

namespace dash {

__global__ void varlen_meta_kernel(const int32_t* __restrict__ cu_seqlens,
                                   int num_seqs, int B,
                                   int32_t* __restrict__ cu_chunks,
                                   int32_t* __restrict__ cu_pad) {
  if (threadIdx.x != 0) return;
  int32_t acc = 0, pad = 0;
  cu_chunks[0] = 0;
  if (cu_pad) cu_pad[0] = 0;
  for (int s = 0; s < num_seqs; ++s) {
    const int32_t L = cu_seqlens[s + 1] - cu_seqlens[s];
    acc += L / B;
    cu_chunks[s + 1] = acc;
    pad += (L + 63) / 64 * 64;
    if (cu_pad) cu_pad[s + 1] = pad;
  }
}

hipError_t launch_varlen_meta(const int32_t* cu_seqlens, int num_seqs, int B,
                              int32_t* cu_chunks, int32_t* cu_pad, hipStream_t st) {
  hipLaunchKernelGGL(varlen_meta_kernel, dim3(1), dim3(64), 0, st, cu_seqlens,
                     num_seqs, B, cu_chunks, cu_pad);
  return hipGetLastError();
}

template <bool BF16, int D>
__global__ __launch_bounds__(64) void summarize_kernel(
    const void* __restrict__ kp, const float* __restrict__ qbar,
    void* __restrict__ kbarp, const int32_t* __restrict__ cu_seqlens,
    const int32_t* __restrict__ cu_chunks, int max_seqlen, int Hkv, int B) {
  constexpr int ESZ = BF16 ? 2 : 4;
  const int c = blockIdx.x, s = blockIdx.y, h = blockIdx.z;
  const SeqInfo si = seq_info(cu_seqlens, cu_chunks, s, max_seqlen, B);
  if ((c + 1) * B > si.len) return;
  const int64_t row0 = si.start + (int64_t)c * B;
  auto row = [&](int key) -> const void* {
    return (const char*)kp + ((row0 + key) * Hkv + h) * (int64_t)D * ESZ;
  };
  const int64_t orow = (si.chunk_off + c) * Hkv + h;
  summarize_chunk<BF16, D>(row, qbar + h * D, B, (char*)kbarp + orow * D * ESZ);
}

// Decode-cache upkeep: one wave per (batch entry b, KV head h), append_token.
template <bool BF16, int D>
__global__ __launch_bounds__(64) void cache_append_kernel(
    Geom g, const void* __restrict__ knew, const void* __restrict__ vnew,
    const int32_t* __restrict__ seqlens, const float* __restrict__ qbar,
    void* __restrict__ kc, void* __restrict__ vc, void* __restrict__ kbar) {
  append_token<BF16, D>(g, knew, vnew, seqlens, qbar, kc, vc, kbar, blockIdx.x, blockIdx.y);
}

// Estimated summary of a position's own, partial chunk: q_bar's phase-0
// attention over the chunk's keys up to the position.  One wave scans keys
// key(0) .. key(len-1) of one chunk in order with a running (max, sum,
// weighted key) in base 2, lane l holding dimensions EPL l .. EPL l + EPL - 1;
// after key t the normalised running value is position t's estimate, written
// to out(t) when ALL (else only after the last key), rounded once.
template <bool BF16, int D, int MAXK, bool ALL, class KeyFn, class OutFn>
__device__ __forceinline__ void diag_scan(KeyFn key, int len, const float* __restrict__ qbar_h,
                                          OutFn out) {
  constexpr int EPL = D / kWave;  // 1 or 2 elements per lane
  const int lane = threadIdx.x;
  float qv[EPL];
#pragma unroll
  for (int e = 0; e < EPL; ++e) qv[e] = qbar_h[EPL * lane + e];
  const float sc = kLog2e / sqrtf((float)D);
  float m = -INFINITY, l = 0.f, acc[EPL];
#pragma unroll
  for (int e = 0; e < EPL; ++e) acc[e] = 0.f;
  // the key's score in log2 units (a wave reduction)
  auto score = [&](const float (&x)[EPL]) -> float {
    float d = 0.f;
#pragma unroll
    for (int e = 0; e < EPL; ++e) d = fmaf(x[e], qv[e], d);
    d = row16_sum(d);
    d += xor16(d);
    d += xor32(d);
    return d * sc;
  };
  // write position t's estimate from the running state
  auto emit = [&](int t) {
    const float inv = 1.f / l;
    char* o = (char*)out(t);
    if constexpr (BF16) {
      if constexpr (EPL == 2)
        *reinterpret_cast<uint32_t*>(o + 4 * lane) = pack_bf16x2(acc[0] * inv, acc[1] * inv);
      else
        *reinterpret_cast<uint16_t*>(o + 2 * lane) = (uint16_t)f32_to_bf16(acc[0] * inv);
    } else {
#pragma unroll
      for (int e = 0; e < EPL; ++e) reinterpret_cast<float*>(o)[EPL * lane + e] = acc[e] * inv;
    }
  };
  // fold key t (its EPL elements in x, score z) into the running state;
  // write out(t)
  auto step = [&](int t, const float (&x)[EPL], float z) {
    const float mn = fmaxf(m, z);
    const float a = exp2f(m - mn);
    const float p = exp2f(z - mn);
    l = l * a + p;
#pragma unroll
    for (int e = 0; e < EPL; ++e) acc[e] = fmaf(p, x[e], acc[e] * a);
    m = mn;
    if (ALL || t == len - 1) emit(t);
  };
  if constexpr (BF16) {
    // every key's elements (one 32- or 16-bit word per lane) are loaded up
    // front, so the scan waits for memory once (len <= MAXK = B); the loads
    // are unconditional, keys past len re-reading key len - 1
    const char* kbase = (const char*)key(0);
    const int64_t kstride = (const char*)key(1) - kbase;
    uint32_t raw[MAXK];
#pragma unroll
    for (int t = 0; t < MAXK; ++t) {
      const char* row = kbase + (int64_t)min(t, len - 1) * kstride;
      raw[t] = EPL == 2 ? *reinterpret_cast<const uint32_t*>(row + 4 * lane)
                        : (uint32_t)*reinterpret_cast<const uint16_t*>(row + 2 * lane);
    }
    __builtin_amdgcn_sched_barrier(0);  // every load issued before the first use
    auto unpack = [&](int t, float (&x)[EPL]) {
      if constexpr (EPL == 2) {
        x[0] = bf16lo(raw[t]);
        x[1] = bf16hi(raw[t]);
      } else {
        x[0] = bf16_to_f32(raw[t]);
      }
    };
    auto lanef = [](float v, int j) {
      return __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), j));
    };
    // 64 keys at a time, key t0 + j in lane j: its score (the same wave
    // reduction per key), the running max after it (a prefix max over the
    // lanes, exact in any order), and so each key's rescale factor
    // a = 2^(m_before - m_after) and weight p = 2^(z - m_after) with two
    // exponentials for all 64 keys.  The sums l and acc then take the keys in
    // order, with the same multiply-adds as a key-by-key running softmax.
#pragma unroll
    for (int t0 = 0; t0 < MAXK; t0 += kWave) {
      if (t0 < len) {
        float zl = -INFINITY;
#pragma unroll
        for (int j = 0; j < kWave; ++j) {
          float x[EPL];
          unpack(t0 + j, x);
          const float z = score(x);
          zl = lane == j ? z : zl;
        }
        if (t0 + lane >= len) zl = -INFINITY;  // (copies of key len - 1)
        float mt = zl;
#pragma unroll
        for (int o = 1; o < kWave; o <<= 1) {
          const float y = __shfl_up(mt, o);
          if (lane >= o) mt = fmaxf(mt, y);
        }
        mt = fmaxf(mt, m);
        float mb = __shfl_up(mt, 1);
        if (lane == 0) mb = m;
        const float av = exp2f(mb - mt);
        const float pv = exp2f(zl - mt);
#pragma unroll
        for (int j = 0; j < kWave; ++j) {
          if (t0 + j < len) {
            const float a = lanef(av, j), pj = lanef(pv, j);
            float x[EPL];
            unpack(t0 + j, x);
            l = l * a + pj;
#pragma unroll
            for (int e = 0; e < EPL; ++e) acc[e] = fmaf(pj, x[e], acc[e] * a);
            if (ALL) emit(t0 + j);
          }
        }
        m = lanef(mt, kWave - 1);
      }
    }
    if (!ALL) emit(len - 1);
  } else {
    constexpr int GRP = 8;  // keys whose loads are issued together
    for (int t0 = 0; t0 < len; t0 += GRP) {
      float xs[GRP][EPL];
#pragma unroll
      for (int j = 0; j < GRP; ++j) {
        const float* row = (const float*)key(min(t0 + j, len - 1));
#pragma unroll
        for (int e = 0; e < EPL; ++e) xs[j][e] = row[EPL * lane + e];
      }
#pragma unroll
      for (int j = 0; j < GRP; ++j) {
        if (t0 + j >= len) break;
        step(t0 + j, xs[j], score(xs[j]));
      }
    }
  }
}

// Prefill: every position's estimate, kdiag [T, Hkv, D]; one wave per
// (chunk, sequence, KV head), the last chunk of a sequence possibly partial.
template <bool BF16, int D, int BB>
__global__ __launch_bounds__(64) void diag_summary_kernel(
    const void* __restrict__ kp, const float* __restrict__ qbar, void* __restrict__ kdiag,
    const int32_t* __restrict__ cu_seqlens, int max_seqlen, int Hkv, int B) {
  constexpr int ESZ = BF16 ? 2 : 4;
  const int c = blockIdx.x, s = blockIdx.y, h = blockIdx.z;
  const SeqInfo si = seq_info(cu_seqlens, nullptr, s, max_seqlen, B);
  const int t0 = c * B;
  if (t0 >= si.len) return;
  const int len = min(B, si.len - t0);
  const int64_t row0 = si.start + t0;
  auto key = [&](int t) -> const void* {
    return (const char*)kp + ((row0 + t) * Hkv + h) * (int64_t)D * ESZ;
  };
  auto out = [&](int t) -> void* {
    return (char*)kdiag + ((row0 + t) * Hkv + h) * (int64_t)D * ESZ;
  };
  diag_scan<BF16, D, BB, true>(key, len, qbar + h * D, out);
}

// Decode: the estimate at each batch entry's new position L-1 from the
// cached keys n B .. L-1 (n = floor((L-1)/B)), kdiag [batch, Hkv, D].
template <bool BF16, int D, int BB>
__global__ __launch_bounds__(64) void decode_diag_kernel(
    const void* __restrict__ kc, const int32_t* __restrict__ seqlens,
    const float* __restrict__ qbar, void* __restrict__ kdiag, int cap, int Hkv, int B) {
  constexpr int ESZ = BF16 ? 2 : 4;
  const int b = blockIdx.x, h = blockIdx.y;
  const int L = seqlens[b];
  const int t0 = ((L - 1) / B) * B;
  const int64_t row0 = (int64_t)b * cap + t0;
  auto key = [&](int t) -> const void* {
    return (const char*)kc + ((row0 + t) * Hkv + h) * (int64_t)D * ESZ;
  };
  auto out = [&](int) -> void* {
    return (char*)kdiag + ((int64_t)b * Hkv + h) * D * ESZ;
  };
  diag_scan<BF16, D, BB, false>(key, L - t0, qbar + h * D, out);
}

hipError_t launch_diag_summary(const Geom& g, const void* k, const float* qbar, void* kdiag,
                               hipStream_t st) {
  const int maxC = (g.max_seqlen + g.B - 1) / g.B;
  if (maxC == 0 || g.num_seqs == 0) return hipSuccess;
  dim3 grid(maxC, g.num_seqs, g.Hkv);
#define DASH_DIAG(BF, DD, BB)                                                               \
  hipLaunchKernelGGL((diag_summary_kernel<BF, DD, BB>), grid, dim3(kWave), 0, st, k, qbar,    \
                     kdiag, g.cu_seqlens, g.max_seqlen, g.Hkv, g.B)
#define DASH_DIAG_B(BF, DD) \
  do { if (g.B == 64) DASH_DIAG(BF, DD, 64); else DASH_DIAG(BF, DD, 128); } while (0)
  if (g.bf16) {
    if (g.D == 64) DASH_DIAG_B(true, 64); else DASH_DIAG_B(true, 128);
  } else {
    if (g.D == 64) DASH_DIAG_B(false, 64); else DASH_DIAG_B(false, 128);
  }
#undef DASH_DIAG_B
#undef DASH_DIAG
  return hipGetLastError();
}

hipError_t launch_decode_diag(const Geom& g, const void* k_cache, const int32_t* seqlens,
                              const float* qbar, void* kdiag, hipStream_t st) {
  if (g.num_seqs == 0) return hipSuccess;
  dim3 grid(g.num_seqs, g.Hkv);
#define DASH_DDIAG(BF, DD, BB)                                                            \
  hipLaunchKernelGGL((decode_diag_kernel<BF, DD, BB>), grid, dim3(kWave), 0, st, k_cache,    \
                     seqlens, qbar, kdiag, g.max_seqlen, g.Hkv, g.B)
#define DASH_DDIAG_B(BF, DD) \
  do { if (g.B == 64) DASH_DDIAG(BF, DD, 64); else DASH_DDIAG(BF, DD, 128); } while (0)
  if (g.bf16) {
    if (g.D == 64) DASH_DDIAG_B(true, 64); else DASH_DDIAG_B(true, 128);
  } else {
    if (g.D == 64) DASH_DDIAG_B(false, 64); else DASH_DDIAG_B(false, 128);
  }
#undef DASH_DDIAG_B
#undef DASH_DDIAG
  return hipGetLastError();
}

hipError_t launch_cache_append(const Geom& g, const void* knew, const void* vnew,
                               const int32_t* seqlens, const float* qbar, void* kc, void* vc,
                               void* kbar, hipStream_t st) {
  if (g.num_seqs == 0) return hipSuccess;
  dim3 grid(g.num_seqs, g.Hkv);
#define DASH_APP(BF, DD)                                                                    \
  hipLaunchKernelGGL((cache_append_kernel<BF, DD>), grid, dim3(kWave), 0, st, g, knew, vnew, \
                     seqlens, qbar, kc, vc, kbar)
  if (g.bf16) {
    if (g.D == 64) DASH_APP(true, 64); else DASH_APP(true, 128);
  } else {
    if (g.D == 64) DASH_APP(false, 64); else DASH_APP(false, 128);
  }
#undef DASH_APP
  return hipGetLastError();
}

hipError_t launch_summarize(const Geom& g, const void* k, const float* qbar,
                            void* kbar, hipStream_t st) {
  const int maxC = g.max_seqlen / g.B;
  if (maxC == 0 || g.num_seqs == 0) return hipSuccess;
  dim3 grid(maxC, g.num_seqs, g.Hkv);
  dim3 block(kWave);
#define DASH_SUM(BF, DD)                                                      \
  hipLaunchKernelGGL((summarize_kernel<BF, DD>), grid, block, 0, st, k, qbar, \
                     kbar, g.cu_seqlens, g.cu_chunks, g.max_seqlen, g.Hkv, g.B)
  if (g.bf16) {
    if (g.D == 64) DASH_SUM(true, 64); else DASH_SUM(true, 128);
  } else {
    if (g.D == 64) DASH_SUM(false, 64); else DASH_SUM(false, 128);
  }
#undef DASH_SUM
  return hipGetLastError();
}

}  // namespace dash
