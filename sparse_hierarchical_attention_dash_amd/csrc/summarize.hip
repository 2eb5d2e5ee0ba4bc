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
  constexpr int EPL = 16 / ESZ;   // elements per 16-byte load
  constexpr int LPR = D / EPL;    // lanes per key row
  constexpr int KPI = kWave / LPR;  // keys per load instruction
  const int c = blockIdx.x, s = blockIdx.y, h = blockIdx.z;
  const SeqInfo si = seq_info(cu_seqlens, cu_chunks, s, max_seqlen, B);
  if ((c + 1) * B > si.len) return;

  const int lane = threadIdx.x;
  const int sub = lane % LPR;
  const int kr = lane / LPR;
  float qv[EPL];
#pragma unroll
  for (int e = 0; e < EPL; ++e) qv[e] = qbar[h * D + sub * EPL + e];
  const float sc = kLog2e / sqrtf((float)D);

  float m = -INFINITY, l = 0.f, acc[EPL];
#pragma unroll
  for (int e = 0; e < EPL; ++e) acc[e] = 0.f;

  const int64_t row0 = si.start + (int64_t)c * B;
  const int iters = B / KPI;
  for (int it = 0; it < iters; ++it) {
    const int key = it * KPI + kr;
    const char* src = (const char*)kp + (((row0 + key) * Hkv + h) * D + sub * EPL) * ESZ;
    const u32x4 raw = ldg16(src);
    float x[EPL];
    if constexpr (BF16) {
#pragma unroll
      for (int w = 0; w < 4; ++w) {
        x[2 * w] = bf16lo(raw[w]);
        x[2 * w + 1] = bf16hi(raw[w]);
      }
    } else {
#pragma unroll
      for (int w = 0; w < 4; ++w) x[w] = __uint_as_float(raw[w]);
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
    const int64_t orow = (si.chunk_off + c) * Hkv + h;
    if constexpr (BF16) {
      u32x4 w;
#pragma unroll
      for (int q = 0; q < 4; ++q)
        w[q] = pack_bf16x2(acc[2 * q] * inv, acc[2 * q + 1] * inv);
      *reinterpret_cast<u32x4*>((char*)kbarp + (orow * D + sub * EPL) * 2) = w;
    } else {
      f32x4 w;
#pragma unroll
      for (int q = 0; q < 4; ++q) w[q] = acc[q] * inv;
      *reinterpret_cast<f32x4*>((char*)kbarp + (orow * D + sub * EPL) * 4) = w;
    }
  }
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
