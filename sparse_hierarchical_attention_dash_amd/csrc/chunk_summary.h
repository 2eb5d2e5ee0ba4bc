// Phase 0 on one chunk, and the decode-cache append built on it ("Fase 0:
// Lokale Chunk Samenvatting" of the gist.science technical summary: a chunk's
// summary is the learned query's local attention over the chunk's keys).
// Shared by the summary kernels and by the decode routing's first pass, which
// runs the append of a fused decode step beside the routing logits.
#pragma once

#include "dash_device.h"
#include "dash_internal.h"

namespace dash {

// One wave summarises one chunk of B keys: key t's row (this KV head, D
// elements) starts at row(t).  Lane group kr (LPR lanes, one key row per load
// instruction) takes keys kr, kr + KPI, ...; each group keeps a running
// (max, sum, weighted key) in base 2, the groups merge by shuffles, and lanes
// 0 .. LPR-1 write the result, rounded once, to out.
template <bool BF16, int D, class RowFn>
__device__ __forceinline__ void summarize_chunk(RowFn row, const float* __restrict__ qbar_h, int B,
                                                void* __restrict__ out) {
  constexpr int ESZ = BF16 ? 2 : 4;
  constexpr int EPL = 16 / ESZ;   // elements per 16-byte load
  constexpr int LPR = D / EPL;    // lanes per key row
  constexpr int KPI = kWave / LPR;  // keys per load instruction
  const int lane = threadIdx.x;
  const int sub = lane % LPR;
  const int kr = lane / LPR;
  float qv[EPL];
#pragma unroll
  for (int e = 0; e < EPL; ++e) qv[e] = qbar_h[sub * EPL + e];
  const float sc = kLog2e / sqrtf((float)D);

  float m = -INFINITY, l = 0.f, acc[EPL];
#pragma unroll
  for (int e = 0; e < EPL; ++e) acc[e] = 0.f;

  // the loads of GRP keys per lane group are issued together, then folded in
  // key order (iters is a multiple of GRP for every supported B, D, dtype)
  constexpr int GRP = 8;
  const int iters = B / KPI;
  for (int it0 = 0; it0 < iters; it0 += GRP) {
    u32x4 raw[GRP];
#pragma unroll
    for (int j = 0; j < GRP; ++j)
      raw[j] = ldg16((const char*)row((it0 + j) * KPI + kr) + sub * EPL * ESZ);
#pragma unroll
    for (int j = 0; j < GRP; ++j) {
      float x[EPL];
      if constexpr (BF16) {
#pragma unroll
        for (int w = 0; w < 4; ++w) {
          x[2 * w] = bf16lo(raw[j][w]);
          x[2 * w + 1] = bf16hi(raw[j][w]);
        }
      } else {
#pragma unroll
        for (int w = 0; w < 4; ++w) x[w] = __uint_as_float(raw[j][w]);
      }
      float d = 0.f;
#pragma unroll
      for (int e = 0; e < EPL; ++e) d = fmaf(x[e], qv[e], d);
#pragma unroll
      for (int o = 1; o < LPR; o <<= 1) d += __shfl_xor(d, o);
      const float z = d * sc;
      const float mn = fmaxf(m, z);
      const float a = exp2f(m - mn);
      const float p = exp2f(z - mn);
      l = l * a + p;
#pragma unroll
      for (int e = 0; e < EPL; ++e) acc[e] = fmaf(p, x[e], acc[e] * a);
      m = mn;
    }
  }
  // merge the KPI key groups
#pragma unroll
  for (int o = LPR; o < kWave; o <<= 1) {
    const float m2 = __shfl_xor(m, o);
    const float l2 = __shfl_xor(l, o);
    const float mn = fmaxf(m, m2);
    const float a1 = exp2f(m - mn), a2 = exp2f(m2 - mn);
    l = l * a1 + l2 * a2;
#pragma unroll
    for (int e = 0; e < EPL; ++e) {
      const float o2 = __shfl_xor(acc[e], o);
      acc[e] = acc[e] * a1 + o2 * a2;
    }
    m = mn;
  }
  if (lane < LPR) {
    const float inv = 1.f / l;
    if constexpr (BF16) {
      u32x4 w;
#pragma unroll
      for (int q = 0; q < 4; ++q)
        w[q] = pack_bf16x2(acc[2 * q] * inv, acc[2 * q + 1] * inv);
      *reinterpret_cast<u32x4*>((char*)out + sub * EPL * 2) = w;
    } else {
      f32x4 w;
#pragma unroll
      for (int q = 0; q < 4; ++q) w[q] = acc[q] * inv;
      *reinterpret_cast<f32x4*>((char*)out + sub * EPL * 4) = w;
    }
  }
}

// Decode-cache upkeep of batch entry b and KV head h, by one wave (lanes
// threadIdx.x = 0 .. 63).  The new token's key and value rows go to position
// L - 1 of the caches (L = seqlens[b], the length after the append); when the
// token completes its chunk (L % B == 0), the chunk's summary is computed and
// cached, with the new key taken from k_new itself (the rows before it from
// the cache), so no lane reads a row another lane is writing.
template <bool BF16, int D>
__device__ __forceinline__ void append_token(const Geom& g, const void* __restrict__ knew,
                                             const void* __restrict__ vnew,
                                             const int32_t* __restrict__ seqlens,
                                             const float* __restrict__ qbar, void* __restrict__ kc,
                                             void* __restrict__ vc, void* __restrict__ kbar,
                                             int b, int h) {
  constexpr int ESZ = BF16 ? 2 : 4;
  constexpr int RB = D * ESZ / 16;  // 16-byte pieces per row
  const int lane = threadIdx.x;
  const int L = seqlens[b];
  const int64_t cap = g.max_seqlen;
  const int64_t src = ((int64_t)b * g.Hkv + h) * D * ESZ;              // byte offset in k_new
  const int64_t dst = (((int64_t)b * cap + (L - 1)) * g.Hkv + h) * D * ESZ;
  if (lane < RB) {
    const u32x4 w = ldg16((const char*)knew + src + lane * 16);
    *reinterpret_cast<u32x4*>((char*)kc + dst + lane * 16) = w;
  } else if (lane < 2 * RB) {
    const int pc = lane - RB;
    const u32x4 w = ldg16((const char*)vnew + src + pc * 16);
    *reinterpret_cast<u32x4*>((char*)vc + dst + pc * 16) = w;
  }
  if (L % g.B != 0) return;
  const int c = L / g.B - 1;
  const int64_t row0 = (int64_t)b * cap + (int64_t)c * g.B;
  const int last = g.B - 1;
  auto row = [&](int key) -> const void* {
    return key == last ? (const char*)knew + src
                       : (const char*)kc + ((row0 + key) * g.Hkv + h) * (int64_t)D * ESZ;
  };
  const int64_t orow = ((int64_t)b * (cap / g.B) + c) * g.Hkv + h;
  summarize_chunk<BF16, D>(row, qbar + h * D, g.B, (char*)kbar + orow * D * ESZ);
}

}  // namespace dash
