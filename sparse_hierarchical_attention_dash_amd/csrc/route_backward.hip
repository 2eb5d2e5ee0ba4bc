// Backward of phases 1 and 0: from the gradient of each active chunk's
// log-prior to the queries, the summaries, the keys and the learned summary
// query.  The pages make the routing differentiable so that the attention's
// gradient reaches the summaries ("Technische Samenvatting: DashAttention",
// Fase 1, Differentieerbaarheid bullet); each step is the derivative of the
// forward step:
//   prior    b_c = sigma log w_bar_c:     dp_c = sigma db_c / (G w_bar_c)
//            (the same for every head of the group: w_bar is their mean)
//   entmax   du_c = r_c (dp_c - rho),  r = p^(2 - alpha) on the support
//            (alpha = 1: r = p),  rho = sum r dp / sum r
//   logits   u_c = gamma s <q, k_bar_c>:  dq += gamma s sum_c du_c k_bar_c,
//            dk_bar_c += gamma s sum over rows and heads of du_c q
//   phase 0  k_bar = sum_t pi_t k_t, pi = softmax(<q_bar, k_t>/sqrt(D)):
//            dz = pi (<dk_bar, k_t> - sum pi <dk_bar, k>),
//            dk_t += pi_t dk_bar + dz_t q_bar / sqrt(D),
//            dq_bar += sum_t dz_t k_t / sqrt(D)
//
// route_bwd_kernel (one workgroup per row and KV head): recomputes the row's
// logits (MFMA) and, from the forward's thresholds, each head's p; forms
// w_bar, dp, and per head r, rho and du (in LDS); adds gamma s du K_bar to
// dq; stores dp (over db) and each head's (threshold, softmax sum, rho) for
// the chunk pass.
// kbar_bwd_kernel (one workgroup per complete chunk and KV head): scans the
// rows that route to the chunk, recomputes their du for it from the stored
// per-head terms, accumulates dk_bar, then runs the summary's backward.
// bf16, G = 16 or 32, fixed-length sequences.
#include "dash_device.h"
#include "dash_internal.h"

namespace dash {

// d^e for d >= 0 (0 at d = 0 unless e = 0, where it is the support indicator)
__device__ __forceinline__ float pow_pos(float d, float e) {
  if (e == 0.f) return d > 0.f ? 1.f : 0.f;
  return d > 0.f ? exp2f(e * __log2f(d)) : 0.f;
}

template <int D, int CP>
__global__ __launch_bounds__(256) void route_bwd_kernel(Geom g, RouteBwdParams p) {
  constexpr int NTH = 256;
  constexpr int KS = D / 32;
  constexpr int USTR = CP + 16;
  __shared__ float U[16 * USTR];   // logits, then du, of one 16-head tile
  __shared__ float Wp[CP];         // sum over the group's heads of p, then dp
  __shared__ float Hp[16][2];      // per head: threshold (x units) or max u; softmax sum
  const int row = blockIdx.x, h = blockIdx.y;
  const int tid = threadIdx.x, lane = tid & 63, wv = tid >> 6;
  const int r = lane & 15, gq = lane >> 4;
  const int64_t T = g.T;
  const int s = row / g.max_seqlen;
  const int pos = row - s * g.max_seqlen;
  const int64_t kb0 = (int64_t)s * (g.max_seqlen / g.B);
  const int n = pos / g.B;
  const int G = g.G;
  float4* sc = p.sc;
  if (n == 0) {
    if (tid < G) sc[(int64_t)(h * G + tid) * T + row] = make_float4(0.f, 0.f, 0.f, 0.f);
    return;
  }
  const float alpha = p.alpha;
  const bool smax = !(alpha > 1.f);
  const float am1 = alpha - 1.f;
  const float ep = smax ? 1.f : 1.f / am1;            // p = d^ep
  const float er = smax ? 1.f : (2.f - alpha) / am1;  // r = d^er
  const int HT = G / 16;

  // logits of head tile ht into U (16 heads x n chunks, MFMA)
  auto logits = [&](int ht) {
    const uint16_t* qrow = (const uint16_t*)p.q + (((int64_t)row * g.Hq + h * G + 16 * ht + r) * D);
    bf16x8 qa[KS];
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) qa[ks] = as_bf16x8(ldg16(qrow + 32 * ks + 8 * gq));
    const int nct = (n + 15) >> 4;
    for (int ct = wv; ct < nct; ct += 4) {
      const int c = min(ct * 16 + r, n - 1);
      const uint16_t* krow = (const uint16_t*)p.kbar + (((kb0 + c) * g.Hkv + h) * (int64_t)D);
      f32x4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int ks = 0; ks < KS; ++ks)
        acc = mfma16x16x32(qa[ks], as_bf16x8(ldg16(krow + 32 * ks + 8 * gq)), acc);
      if (ct * 16 + r < n) {
#pragma unroll
        for (int j = 0; j < 4; ++j) U[(4 * gq + j) * USTR + ct * 16 + r] = acc[j] * p.gamma_scale;
      }
    }
  };
  // per-head threshold (x units) or (max, softmax sum) into Hp; 16 lanes per head
  auto head_params = [&](int ht) {
    const int hh = wv * 4 + (lane >> 4);  // 4 heads per wave
    const float* ur = U + hh * USTR;
    const int qh = h * G + 16 * ht + hh;
    if (smax) {
      float mx = -INFINITY;
      for (int c = r; c < n; c += 16) mx = fmaxf(mx, ur[c]);
      mx = row16_max(mx);
      float z = 0.f;
      for (int c = r; c < n; c += 16) z += exp2f((ur[c] - mx) * kLog2e);
      z = row16_sum(z);
      if (r == 0) { Hp[hh][0] = mx; Hp[hh][1] = z; }
    } else if (r == 0) {
      Hp[hh][0] = p.tau[(int64_t)qh * T + row] * am1;
      Hp[hh][1] = 0.f;
    }
  };
  auto prob = [&](float u, int hh) -> float {
    return smax ? exp2f((u - Hp[hh][0]) * kLog2e) / Hp[hh][1] : pow_pos(u * am1 - Hp[hh][0], ep);
  };
  auto rterm = [&](float u, int hh) -> float {
    return smax ? exp2f((u - Hp[hh][0]) * kLog2e) / Hp[hh][1] : pow_pos(u * am1 - Hp[hh][0], er);
  };

  // ---- pass 1: w_bar (as G w_bar) over all head tiles
  for (int c = tid; c < n; c += NTH) Wp[c] = 0.f;
  for (int ht = 0; ht < HT; ++ht) {
    __syncthreads();
    logits(ht);
    __syncthreads();
    head_params(ht);
    __syncthreads();
    for (int c = tid; c < n; c += NTH) {
      float w = 0.f;
#pragma unroll 4
      for (int hh = 0; hh < 16; ++hh) w += prob(U[hh * USTR + c], hh);
      Wp[c] += w;
    }
  }
  __syncthreads();
  // ---- dp on the active chunks (written over db)
  const unsigned long long* mrow = p.mask + ((int64_t)h * T + row) * g.W;
  float* drow = p.db + ((int64_t)h * T + row) * g.C_slots;
  for (int c = tid; c < n; c += NTH) {
    const bool on = (mrow[c >> 6] >> (c & 63)) & 1ull;
    const float dp = on ? p.sigma * drow[c] / Wp[c] : 0.f;
    Wp[c] = dp;
    drow[c] = dp;
  }
  // ---- pass 2 per head tile: r, rho, du; dq += gamma s du K_bar
  for (int ht = 0; ht < HT; ++ht) {
    __syncthreads();
    if (HT > 1) {
      logits(ht);
      __syncthreads();
      head_params(ht);
      __syncthreads();
    }
    {
      const int hh = wv * 4 + (lane >> 4);
      float* ur = U + hh * USTR;
      float num = 0.f, den = 0.f;
      for (int c = r; c < n; c += 16) {
        const float rr = rterm(ur[c], hh);
        num = fmaf(rr, Wp[c], num);
        den += rr;
      }
      num = row16_sum(num);
      den = row16_sum(den);
      const float rho = den > 0.f ? num / den : 0.f;
      // every lane of the head has read its U entries above; du overwrites them
      for (int c = r; c < n; c += 16) {
        const float rr = rterm(ur[c], hh);
        ur[c] = rr * (Wp[c] - rho);
      }
      if (r == 0)
        sc[(int64_t)(h * G + 16 * ht + hh) * T + row] = make_float4(Hp[hh][0], Hp[hh][1], rho, 0.f);
    }
    __syncthreads();
    // thread (head hh, dims 8 j .. 8 j + 7) for D = 128 (4 dims for D = 64)
    constexpr int DPT = D / 16;
    const int hh = tid >> 4, j = tid & 15;
    float acc[DPT];
#pragma unroll
    for (int e = 0; e < DPT; ++e) acc[e] = 0.f;
    const float* ur = U + hh * USTR;
    for (int c = 0; c < n; ++c) {
      const float du = ur[c];
      if (du == 0.f) continue;  // off every head's support (wave-divergent skip)
      const uint16_t* krow =
          (const uint16_t*)p.kbar + (((kb0 + c) * g.Hkv + h) * (int64_t)D) + DPT * j;
      if constexpr (DPT == 8) {
        const u32x4 kv = ldg16(krow);
#pragma unroll
        for (int w = 0; w < 4; ++w) {
          acc[2 * w] = fmaf(du, bf16lo(kv[w]), acc[2 * w]);
          acc[2 * w + 1] = fmaf(du, bf16hi(kv[w]), acc[2 * w + 1]);
        }
      } else {
        const u32x2 kv = *reinterpret_cast<const u32x2*>(krow);
#pragma unroll
        for (int w = 0; w < 2; ++w) {
          acc[2 * w] = fmaf(du, bf16lo(kv[w]), acc[2 * w]);
          acc[2 * w + 1] = fmaf(du, bf16hi(kv[w]), acc[2 * w + 1]);
        }
      }
    }
    float* dq = p.dq + ((int64_t)row * g.Hq + h * G + 16 * ht + hh) * D + DPT * j;
#pragma unroll
    for (int e = 0; e < DPT; ++e) dq[e] += p.gamma_scale * acc[e];
  }
}

template <int D, int HT>
__global__ __launch_bounds__(256) void kbar_bwd_kernel(Geom g, RouteBwdParams p) {
  constexpr int NTH = 256;
  constexpr int G = 16 * HT;
  constexpr int DPT = D / 16;        // dims per thread in the (head, dims) layout
  __shared__ float Kb[D];            // the chunk's summary (fp32)
  __shared__ float Qs[G * D];        // one row's queries of the group
  __shared__ float Du[G];
  __shared__ float Acc[16][D];       // dk_bar partial sums, per head-row of threads
  __shared__ int Rows[NTH];
  __shared__ int Wcnt[NTH / 64];
  __shared__ float Red[NTH];
  const int c = blockIdx.x, s = blockIdx.y, h = blockIdx.z;
  const int tid = threadIdx.x, lane = tid & 63, wv = tid >> 6;
  const int len = g.max_seqlen;
  if ((c + 1) * g.B > len) return;   // complete chunks only
  const int64_t T = g.T;
  const int64_t start = (int64_t)s * len;
  const int64_t kbrow = ((int64_t)s * (len / g.B) + c) * g.Hkv + h;
  for (int d = tid; d < D; d += NTH)
    Kb[d] = bf16_to_f32(((const uint16_t*)p.kbar)[kbrow * D + d]);
  const int hh = tid >> 4, j = tid & 15;   // thread (head row, dims DPT j ..)
  float acc[DPT];
#pragma unroll
  for (int e = 0; e < DPT; ++e) acc[e] = 0.f;
  const float am1 = p.alpha - 1.f;
  const bool smax = !(p.alpha > 1.f);
  const float er = smax ? 1.f : (2.f - p.alpha) / am1;
  __syncthreads();

  for (int r0 = (c + 1) * g.B; r0 < len; r0 += NTH) {
    const int i = r0 + tid;
    bool on = false;
    if (i < len) {
      const unsigned long long w = p.mask[((int64_t)h * T + start + i) * g.W + (c >> 6)];
      on = (w >> (c & 63)) & 1ull;
    }
    const uint64_t bal = __ballot(on);
    if (lane == 0) Wcnt[wv] = __popcll(bal);
    __syncthreads();
    int before = 0, total = 0;
#pragma unroll
    for (int w = 0; w < NTH / 64; ++w) {
      before += w < wv ? Wcnt[w] : 0;
      total += Wcnt[w];
    }
    if (on) Rows[before + __popcll(bal & ((1ull << lane) - 1ull))] = i;
    __syncthreads();
    for (int k = 0; k < total; ++k) {
      const int64_t tok = start + Rows[k];
      for (int e = tid; e < G * D; e += NTH)
        Qs[e] = bf16_to_f32(((const uint16_t*)p.q)[(tok * g.Hq + h * G) * D + e]);
      __syncthreads();
      // du of each head for this chunk: u = gamma s <q, k_bar>, r, dp - rho
      for (int q = wv; q < G; q += NTH / 64) {
        float d = 0.f;
        for (int e = lane; e < D; e += 64) d = fmaf(Qs[q * D + e], Kb[e], d);
        d = row16_sum(d);
        d += xor16(d);
        d += xor32(d);
        if (lane == 0) {
          const float u = d * p.gamma_scale;
          const float4 t = p.sc[(int64_t)(h * G + q) * T + tok];
          const float rr = smax ? exp2f((u - t.x) * kLog2e) / t.y : pow_pos(u * am1 - t.x, er);
          const float dp = p.db[((int64_t)h * T + tok) * g.C_slots + c];
          Du[q] = rr * (dp - t.z);
        }
      }
      __syncthreads();
      // dk_bar partial: heads hh, hh + 16 (G = 32), dims DPT j ..
#pragma unroll
      for (int t2 = 0; t2 < HT; ++t2) {
        const int q = hh + 16 * t2;
        const float du = Du[q];
#pragma unroll
        for (int e = 0; e < DPT; ++e) acc[e] = fmaf(du, Qs[q * D + DPT * j + e], acc[e]);
      }
      __syncthreads();
    }
  }
  // dk_bar = gamma s * (sum over the 16 head rows of threads)
#pragma unroll
  for (int e = 0; e < DPT; ++e) Acc[hh][DPT * j + e] = acc[e];
  __syncthreads();
  __shared__ float Dkb[D];
  for (int d = tid; d < D; d += NTH) {
    float t = 0.f;
#pragma unroll
    for (int q = 0; q < 16; ++q) t += Acc[q][d];
    Dkb[d] = t * p.gamma_scale;
  }
  __syncthreads();

  // ---- the summary's backward over the chunk's B keys (thread t: key t)
  const int B = g.B;
  const float sD = 1.f / sqrtf((float)D);
  const float* qb = p.qbar + h * D;
  float z = -INFINITY, dpi = 0.f;
  const uint16_t* krow = nullptr;
  if (tid < B) {
    krow = (const uint16_t*)p.k + ((start + (int64_t)c * B + tid) * g.Hkv + h) * D;
    float a = 0.f, b = 0.f;
    for (int e = 0; e < D; e += 8) {
      const u32x4 kv = ldg16(krow + e);
#pragma unroll
      for (int w = 0; w < 4; ++w) {
        const float x0 = bf16lo(kv[w]), x1 = bf16hi(kv[w]);
        a = fmaf(x0, qb[e + 2 * w], a);
        a = fmaf(x1, qb[e + 2 * w + 1], a);
        b = fmaf(x0, Dkb[e + 2 * w], b);
        b = fmaf(x1, Dkb[e + 2 * w + 1], b);
      }
    }
    z = a * sD;
    dpi = b;
  }
  // softmax over the chunk's keys (block reductions through Red)
  Red[tid] = z;
  __syncthreads();
  for (int o = NTH / 2; o > 0; o >>= 1) {
    if (tid < o) Red[tid] = fmaxf(Red[tid], Red[tid + o]);
    __syncthreads();
  }
  const float zmax = Red[0];
  __syncthreads();
  const float ez = tid < B ? __expf(z - zmax) : 0.f;
  Red[tid] = ez;
  __syncthreads();
  for (int o = NTH / 2; o > 0; o >>= 1) {
    if (tid < o) Red[tid] += Red[tid + o];
    __syncthreads();
  }
  const float zsum = Red[0];
  __syncthreads();
  const float pi = ez / zsum;
  Red[tid] = pi * dpi;
  __syncthreads();
  for (int o = NTH / 2; o > 0; o >>= 1) {
    if (tid < o) Red[tid] += Red[tid + o];
    __syncthreads();
  }
  const float pdp = Red[0];
  __syncthreads();
  const float dz = pi * (dpi - pdp);
  // dk_t += pi_t dk_bar + sD dz_t q_bar (the key rows of this chunk and head
  // belong to this workgroup alone)
  if (tid < B) {
    float* dkr = p.dk + ((start + (int64_t)c * B + tid) * g.Hkv + h) * D;
    for (int e = 0; e < D; ++e) dkr[e] += pi * Dkb[e] + sD * dz * qb[e];
  }
  // dq_bar += sD sum_t dz_t k_t: thread d sums over the keys through LDS
  Red[tid] = dz;
  __syncthreads();
  for (int d = tid; d < D; d += NTH) {
    float t = 0.f;
    for (int kk = 0; kk < B; ++kk)
      t = fmaf(Red[kk], bf16_to_f32(((const uint16_t*)p.k)[((start + (int64_t)c * B + kk) * g.Hkv + h) * D + d]), t);
    atomicAdd(&p.dqbar[h * D + d], sD * t);
  }
}

hipError_t launch_route_bwd(const Geom& g, const RouteBwdParams& p, hipStream_t st) {
  if (g.T == 0) return hipSuccess;
  dim3 grid((unsigned)g.T, g.Hkv);
#define DASH_RB(DD, CPV) hipLaunchKernelGGL((route_bwd_kernel<DD, CPV>), grid, dim3(256), 0, st, g, p)
#define DASH_RB_CP(DD)                                  \
  do {                                                  \
    if (g.C_slots <= 256) DASH_RB(DD, 256);             \
    else if (g.C_slots <= 512) DASH_RB(DD, 512);        \
    else if (g.C_slots <= 1024) DASH_RB(DD, 1024);      \
    else DASH_RB(DD, 2048);                             \
  } while (0)
  if (g.D == 64) DASH_RB_CP(64); else DASH_RB_CP(128);
#undef DASH_RB_CP
#undef DASH_RB
  const int C = g.max_seqlen / g.B;
  if (C == 0) return hipGetLastError();
  dim3 cgrid(C, g.num_seqs, g.Hkv);
#define DASH_KB(DD, HH) hipLaunchKernelGGL((kbar_bwd_kernel<DD, HH>), cgrid, dim3(256), 0, st, g, p)
  if (g.G == 16) {
    if (g.D == 64) DASH_KB(64, 1); else DASH_KB(128, 1);
  } else {
    if (g.D == 64) DASH_KB(64, 2); else DASH_KB(128, 2);
  }
#undef DASH_KB
  return hipGetLastError();
}

}  // namespace dash
