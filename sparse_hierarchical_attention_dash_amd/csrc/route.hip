// Phase 1: alpha-entmax chunk routing ("Fase 1: Entmax Chunk Routering" of the
// gist.science technical summary, equation w_hat = alpha-entmax(gamma z_bar),
// and its GQA bullet: the routing probabilities of the query heads that share a
// KV head are averaged into one shared support).
//
// One workgroup (4 waves) per (token row, KV head):
//   1. logits u[q][c] = gamma*s*<q_q, k_bar_c> for the G query heads of the
//      group and the n = floor(i/B) routable chunks, computed 16 heads x 16
//      chunks at a time with bf16 MFMA (fp32 accumulate; products of bf16 are
//      exact in fp32) and kept in LDS only, never in HBM;
//   2. per head, the entmax threshold tau with x = (alpha-1) u: Newton's method
//      on the convex, decreasing mass f(t) = sum_c [x_c - t]_+^(1/(alpha-1))
//      started at t0 = max(x) - 1 (where f >= 1) moves monotonically up to the
//      root; for alpha = 2 (sparsemax) and alpha = 1.5 the threshold is then
//      recomputed in closed form on the support found and kept if consistent;
//   3. w_bar_c = (1/G) sum_q [x_qc - tau_q]_+^(1/(alpha-1)), the active bit
//      OR_q [x_qc > tau_q] gathered 64 chunks per wave with a ballot into one
//      mask word, and log_prior_c = sigma*log(w_bar_c) on the active chunks.
// alpha = 1 is softmax routing: every routable chunk is active.
#include "dash_device.h"
#include "dash_internal.h"

namespace dash {

// d^e and d^(e-1) for d > 0; e = 1, 2, 4 exactly, anything else via exp2/log2.
__device__ __forceinline__ void pow_pair(float d, float e, int ecls, float& pw,
                                         float& pd) {
  if (ecls == 1) {
    pw = d;
    pd = 1.f;
  } else if (ecls == 2) {
    pw = d * d;
    pd = d;
  } else if (ecls == 4) {
    const float d2 = d * d;
    pw = d2 * d2;
    pd = d2 * d;
  } else {
    const float lg = __log2f(d);
    pw = exp2f(e * lg);
    pd = exp2f((e - 1.f) * lg);
  }
}

__device__ __forceinline__ float pow_e(float d, float e, int ecls) {
  if (ecls == 1) return d;
  if (ecls == 2) return d * d;
  if (ecls == 4) {
    const float d2 = d * d;
    return d2 * d2;
  }
  return exp2f(e * __log2f(d));
}

// Threshold (x units) of one row whose values xs live in the wave's registers,
// chunk c = lane + 64k; entries past the row are -inf.
template <int NK>
__device__ float solve_tau(const float (&xs)[NK], float xmax, float e, int ecls) {
  float tau = xmax - 1.f;  // the top entry alone has mass 1 here
  for (int it = 0; it < 200; ++it) {
    float f = 0.f, gd = 0.f;
#pragma unroll
    for (int k = 0; k < NK; ++k) {
      const float d = xs[k] - tau;
      if (d > 0.f) {
        float pw, pd;
        pow_pair(d, e, ecls, pw, pd);
        f += pw;
        gd += pd;
      }
    }
    f = wave_sum(f);
    gd = wave_sum(gd);
    const float step = (f - 1.f) / (e * gd);
    const float nt = tau + step;
    if (!(step > 0.f) || nt == tau) break;
    tau = nt;
    if (step <= 1e-7f * fmaxf(1.f, fabsf(tau))) break;
  }
  if (ecls == 1 || ecls == 2) {
    // closed form on the support S = {x > tau}: sparsemax tau = (sum_S x - 1)/|S|;
    // 1.5-entmax tau = M - sqrt((1 - sum_S (x-M)^2)/|S|), M the mean over S
    float s1 = 0.f, cnt = 0.f, mn_in = INFINITY, mx_out = -INFINITY;
#pragma unroll
    for (int k = 0; k < NK; ++k) {
      if (xs[k] > tau) {
        s1 += xs[k];
        cnt += 1.f;
        mn_in = fminf(mn_in, xs[k]);
      } else {
        mx_out = fmaxf(mx_out, xs[k]);
      }
    }
    s1 = wave_sum(s1);
    cnt = wave_sum(cnt);
    mn_in = wave_min(mn_in);
    mx_out = wave_max(mx_out);
    float t2;
    if (ecls == 1) {
      t2 = (s1 - 1.f) / cnt;
    } else {
      const float M = s1 / cnt;
      float q2 = 0.f;
#pragma unroll
      for (int k = 0; k < NK; ++k) {
        if (xs[k] > tau) {
          const float d = xs[k] - M;
          q2 = fmaf(d, d, q2);
        }
      }
      q2 = wave_sum(q2);
      t2 = M - sqrtf(fmaxf(0.f, (1.f - q2) / cnt));
    }
    if (cnt > 0.f && t2 < mn_in && t2 >= mx_out) tau = t2;
  }
  return tau;
}

template <bool BF16, int D, int CP>
__global__ __launch_bounds__(256) void route_kernel(Geom g, RouteParams p) {
  constexpr int NK = CP / kWave;
  __shared__ float U[16][CP];       // logits of one 16-head tile
  __shared__ float Wsum[CP];        // sum over the group's heads of p
  __shared__ uint64_t Bits[NK];     // active bits
  __shared__ float TauX[16];        // threshold (x units), or max u (softmax)
  __shared__ float Zs[16];          // softmax denominator (alpha = 1)

  const int64_t row = blockIdx.x;
  const int h = blockIdx.y;
  const int tid = threadIdx.x, lane = tid & 63, wv = tid >> 6;
  const int64_t rows = p.rows;

  int64_t tok;   // row of q and of the outputs
  int pos;       // position inside its sequence
  int64_t kb0;   // first summary row of the sequence
  float alpha = p.alpha;
  if (p.seqlens) {
    tok = row;
    pos = p.seqlens[row] - 1;
    kb0 = row * (int64_t)(g.max_seqlen / g.B);
  } else {
    const int s = g.cu_seqlens ? find_seq(g.cu_seqlens, g.num_seqs, row)
                               : (int)(row / g.max_seqlen);
    const SeqInfo si = seq_info(g.cu_seqlens, g.cu_chunks, s, g.max_seqlen, g.B);
    tok = row;
    pos = (int)(row - si.start);
    kb0 = si.chunk_off;
    if (p.alpha_per_seq) alpha = p.alpha_per_seq[s];
  }
  const int n = pos / g.B;
  uint64_t* mrow = p.mask + ((int64_t)h * rows + tok) * g.W;
  if (n <= 0) {
    for (int w = tid; w < g.W; w += 256) mrow[w] = 0ull;
    if (p.tau)
      for (int q = tid; q < g.G; q += 256)
        p.tau[(int64_t)(h * g.G + q) * rows + tok] = INFINITY;
    return;
  }
  const bool smax = !(alpha > 1.f);
  const float am1 = alpha - 1.f;
  const float ex = smax ? 1.f : 1.f / am1;
  const int ecls = smax ? 0 : (ex == 1.f ? 1 : (ex == 2.f ? 2 : (ex == 4.f ? 4 : 0)));
  const float xs_scale = smax ? 1.f : am1;

  for (int c = tid; c < n; c += 256) Wsum[c] = 0.f;
  for (int w = tid; w < NK; w += 256) Bits[w] = 0ull;

  const int ntile_h = (g.G + 15) / 16;
  for (int ht = 0; ht < ntile_h; ++ht) {
    const int h0 = ht * 16;
    const int nh = min(16, g.G - h0);
    __syncthreads();
    // ---- 1. logits
    if constexpr (BF16) {
      const int r = lane & 15, gq = lane >> 4;
      bf16x8 qa[D / 32];
      const uint16_t* qrow =
          (const uint16_t*)p.q + ((tok * g.Hq + h * g.G + h0 + r) * (int64_t)D);
#pragma unroll
      for (int ks = 0; ks < D / 32; ++ks) {
        u32x4 v = {0u, 0u, 0u, 0u};
        if (r < nh) v = ldg16(qrow + 32 * ks + 8 * gq);
        qa[ks] = as_bf16x8(v);
      }
      const int nct = (n + 15) >> 4;
      for (int ct = wv; ct < nct; ct += 4) {
        const int c = ct * 16 + r;
        const uint16_t* krow =
            (const uint16_t*)p.kbar + (((kb0 + c) * g.Hkv + h) * (int64_t)D);
        f32x4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int ks = 0; ks < D / 32; ++ks) {
          u32x4 v = {0u, 0u, 0u, 0u};
          if (c < n) v = ldg16(krow + 32 * ks + 8 * gq);
          acc = mfma16x16x32(qa[ks], as_bf16x8(v), acc);
        }
        if (c < n) {
#pragma unroll
          for (int j = 0; j < 4; ++j) U[4 * gq + j][c] = acc[j] * p.gamma_scale;
        }
      }
    } else {
      for (int idx = tid; idx < nh * n; idx += 256) {
        const int hh = idx / n, c = idx - hh * n;
        const float* qr = (const float*)p.q + ((tok * g.Hq + h * g.G + h0 + hh) * (int64_t)D);
        const float* kr = (const float*)p.kbar + (((kb0 + c) * g.Hkv + h) * (int64_t)D);
        float d = 0.f;
#pragma unroll 8
        for (int e = 0; e < D; e += 4) {
          const f32x4 a4 = *reinterpret_cast<const f32x4*>(qr + e);
          const f32x4 b4 = *reinterpret_cast<const f32x4*>(kr + e);
          d = fmaf(a4[0], b4[0], d);
          d = fmaf(a4[1], b4[1], d);
          d = fmaf(a4[2], b4[2], d);
          d = fmaf(a4[3], b4[3], d);
        }
        U[hh][c] = d * p.gamma_scale;
      }
    }
    __syncthreads();
    // ---- 2. thresholds, one head per wave at a time
    for (int hh = wv; hh < nh; hh += 4) {
      float xs[NK];
      float xmax = -INFINITY;
#pragma unroll
      for (int k = 0; k < NK; ++k) {
        const int c = lane + 64 * k;
        const float x = (c < n) ? U[hh][c] * xs_scale : -INFINITY;
        xs[k] = x;
        xmax = fmaxf(xmax, x);
      }
      xmax = wave_max(xmax);
      if (smax) {
        float z = 0.f;
#pragma unroll
        for (int k = 0; k < NK; ++k) z += exp2f((xs[k] - xmax) * kLog2e);
        z = wave_sum(z);
        if (lane == 0) {
          TauX[hh] = xmax;
          Zs[hh] = z;
        }
      } else {
        const float tau = solve_tau<NK>(xs, xmax, ex, ecls);
        if (lane == 0) TauX[hh] = tau;
      }
    }
    __syncthreads();
    if (p.tau && tid < nh)
      p.tau[(int64_t)(h * g.G + h0 + tid) * rows + tok] =
          smax ? -INFINITY : TauX[tid] / am1;
    // ---- 3. group weight numerators and active bits
    for (int base = 0; base < n; base += 256) {
      const int c = base + tid;
      bool on = false;
      if (c < n) {
        float ws = 0.f;
        for (int hh = 0; hh < nh; ++hh) {
          if (smax) {
            ws += exp2f((U[hh][c] - TauX[hh]) * kLog2e) / Zs[hh];
            on = true;
          } else {
            const float d = U[hh][c] * am1 - TauX[hh];
            if (d > 0.f) {
              on = true;
              ws += pow_e(d, ex, ecls);
            }
          }
        }
        Wsum[c] += ws;
      }
      const uint64_t b = __ballot(on);
      if (lane == 0) Bits[(base >> 6) + wv] |= b;
    }
  }
  __syncthreads();
  if (p.log_prior) {
    float* lrow = p.log_prior + ((int64_t)h * rows + tok) * g.C_slots;
    const float invG = 1.f / (float)g.G;
    for (int c = tid; c < n; c += 256) {
      const bool on = (Bits[c >> 6] >> (c & 63)) & 1ull;
      float v = -INFINITY;
      if (on) v = (p.sigma == 0.f) ? 0.f : p.sigma * logf(fmaxf(Wsum[c] * invG, 1e-38f));
      lrow[c] = v;
    }
  }
  for (int w = tid; w < g.W; w += 256) mrow[w] = (w < NK) ? Bits[w] : 0ull;
}

hipError_t launch_route(const Geom& g, const RouteParams& p, hipStream_t st) {
  if (p.rows == 0) return hipSuccess;
  dim3 grid((unsigned)p.rows, g.Hkv);
  dim3 block(256);
#define DASH_ROUTE(BF, DD, CPV)                                                   \
  hipLaunchKernelGGL((route_kernel<BF, DD, CPV>), grid, block, 0, st, g, p)
#define DASH_ROUTE_CP(BF, DD)                                                     \
  do {                                                                            \
    if (g.C_slots <= 256) DASH_ROUTE(BF, DD, 256);                                \
    else if (g.C_slots <= 512) DASH_ROUTE(BF, DD, 512);                           \
    else if (g.C_slots <= 1024) DASH_ROUTE(BF, DD, 1024);                         \
    else DASH_ROUTE(BF, DD, 2048);                                                \
  } while (0)
  if (g.bf16) {
    if (g.D == 64) DASH_ROUTE_CP(true, 64); else DASH_ROUTE_CP(true, 128);
  } else {
    if (g.D == 64) DASH_ROUTE_CP(false, 64); else DASH_ROUTE_CP(false, 128);
  }
#undef DASH_ROUTE_CP
#undef DASH_ROUTE
  return hipGetLastError();
}

}  // namespace dash
