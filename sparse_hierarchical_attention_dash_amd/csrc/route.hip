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
//   2. per head (16 lanes per head, 4 heads per wave solved side by side with
//      DPP row reductions), the entmax threshold tau with x = (alpha-1) u: Newton's method
//      on the convex, decreasing mass f(t) = sum_c [x_c - t]_+^(1/(alpha-1))
//      started at t0 = max(x) - 1 (where f >= 1) moves monotonically up to the
//      root; for alpha = 2 (sparsemax) and alpha = 1.5 the threshold is then
//      recomputed in closed form on the support found and kept if consistent;
//   3. w_bar_c = (1/G) sum_q [x_qc - tau_q]_+^(1/(alpha-1)), the active bit
//      OR_q [x_qc > tau_q] gathered 64 chunks per wave with a ballot into one
//      mask word, and log_prior_c = sigma*log(w_bar_c) on the active chunks.
// alpha = 1 is softmax routing: every routable chunk is active.
//
// Top-k routing (topk > 0; the fixed-size block selection of the hierarchical
// methods the pages compare against, NSA and InfLLMv2: the top-k blocks by
// coarse attention scores, then plain softmax attention over them): each
// head's softmax over the routable chunks, summed over the group's heads, is
// the chunk's score; the min(k, n) chunks of highest score are active (ties
// to the lower chunk index), with bias 0.
#include <algorithm>
#include <type_traits>

#include "chunk_summary.h"
#include "dash_device.h"
#include "dash_internal.h"

namespace dash {

// d^e and d^(e-1) for d >= 0 without branches; e = 1, 2, 4 exactly (ECLS),
// anything else (ECLS = 0) via exp2(e log2 d), which is 0 at d = 0.
template <int ECLS>
__device__ __forceinline__ void pow_pair(float d, float e, float& pw, float& pd) {
  if constexpr (ECLS == 1) {
    pw = d;
    pd = d > 0.f ? 1.f : 0.f;
  } else if constexpr (ECLS == 2) {
    pw = d * d;
    pd = d;
  } else if constexpr (ECLS == 4) {
    const float d2 = d * d;
    pw = d2 * d2;
    pd = d2 * d;
  } else {
    const float lg = __log2f(d);
    pw = exp2f(e * lg);
    pd = exp2f((e - 1.f) * lg);
  }
}

// Reductions over the LPH lanes that hold one head's row (LPH = 16: one DPP
// row; 32 or 64: rows joined by cross-row exchanges).
template <int LPH>
__device__ __forceinline__ float head_sum(float v) {
  v = row16_sum(v);
  if constexpr (LPH >= 32) v += xor16(v);
  if constexpr (LPH == 64) v += xor32(v);
  return v;
}
template <int LPH>
__device__ __forceinline__ float head_max(float v) {
  v = row16_max(v);
  if constexpr (LPH >= 32) v = fmaxf(v, xor16(v));
  if constexpr (LPH == 64) v = fmaxf(v, xor32(v));
  return v;
}
template <int LPH>
__device__ __forceinline__ float head_min(float v) {
  v = row16_min(v);
  if constexpr (LPH >= 32) v = fminf(v, xor16(v));
  if constexpr (LPH == 64) v = fminf(v, xor32(v));
  return v;
}

// Threshold (x units) of one routing row held by LPH lanes in xs[k] (entries
// past the row are -1e30); xout is the largest value of the row left out of
// xs (all at or below xmax - 1, so never in the support), -inf if none.  The
// rows of a wave (64/LPH query heads) iterate together; a converged row
// keeps its threshold while the others finish.  Branch-free per element:
// d = max(x - tau, 0) contributes nothing off the support.
template <int NK, int LPH, int ECLS>
__device__ float solve_tau_row(const float (&xs)[NK], float xmax, float e, bool live,
                               float xout) {
  float tau = xmax - 1.f;  // the top entry alone has mass 1 here
  bool done = !live;
  for (int it = 0; it < 200; ++it) {
    if (__ballot(!done) == 0ull) break;
    float f = 0.f, gd = 0.f;
#pragma unroll
    for (int k = 0; k < NK; ++k) {
      const float d = fmaxf(xs[k] - tau, 0.f);
      float pw, pd;
      pow_pair<ECLS>(d, e, pw, pd);
      f += pw;
      gd += pd;
    }
    f = head_sum<LPH>(f);
    gd = head_sum<LPH>(gd);
    if (!done) {
      const float step = (f - 1.f) / (e * gd);
      const float nt = tau + step;
      if (!(step > 0.f) || nt == tau) {
        done = true;
      } else {
        tau = nt;
        if (step <= 1e-7f * fmaxf(1.f, fabsf(tau))) done = true;
      }
    }
  }
  if constexpr (ECLS == 1 || ECLS == 2) {
    // closed form on the support S = {x > tau}: sparsemax tau = (sum_S x - 1)/|S|;
    // 1.5-entmax tau = M - sqrt((1 - sum_S (x-M)^2)/|S|), M the mean over S
    float s1 = 0.f, cnt = 0.f, mn_in = INFINITY, mx_out = -INFINITY;
#pragma unroll
    for (int k = 0; k < NK; ++k) {
      const bool in = xs[k] > tau;
      s1 += in ? xs[k] : 0.f;
      cnt += in ? 1.f : 0.f;
      mn_in = fminf(mn_in, in ? xs[k] : INFINITY);
      mx_out = fmaxf(mx_out, in ? -INFINITY : xs[k]);
    }
    s1 = head_sum<LPH>(s1);
    cnt = head_sum<LPH>(cnt);
    mn_in = head_min<LPH>(mn_in);
    mx_out = fmaxf(head_max<LPH>(mx_out), xout);
    float t2;
    if constexpr (ECLS == 1) {
      t2 = (s1 - 1.f) / cnt;
    } else {
      const float M = s1 / cnt;
      float q2 = 0.f;
      // recompare below rather than keep NK lane masks alive across the sums
      float tq = tau;
      asm volatile("" : "+v"(tq));
#pragma unroll
      for (int k = 0; k < NK; ++k) {
        const float dm = xs[k] > tq ? xs[k] - M : 0.f;
        q2 = fmaf(dm, dm, q2);
      }
      q2 = head_sum<LPH>(q2);
      t2 = M - sqrtf(fmaxf(0.f, (1.f - q2) / cnt));
    }
    if (live && cnt > 0.f && t2 < mn_in && t2 >= mx_out) tau = t2;
  }
  return tau;
}

constexpr float kFar = -1e30f;  // "not a routable chunk" in the threshold solve

// Inclusive prefix sum over the LPH lanes of a head row.
template <int LPH>
__device__ __forceinline__ int head_scan(int v, int li) {
#pragma unroll
  for (int o = 1; o < LPH; o <<= 1) {
    const int y = __shfl_up(v, o, LPH);
    if (li >= o) v += y;
  }
  return v;
}

// Threshold of routing row hh (LPH lanes; chunk c = li + LPH k of U's row in
// xs[k], k < NKE, where NKE * LPH covers the row's n chunks): x = xs_scale * u;
// U's entries from n to NKE * LPH hold kFar.  Writes TauX[hh] (or, for softmax
// routing, the row max and the denominator).
// The threshold is at least xmax - 1 (the top entry alone has mass 1 there),
// so only the candidates x > xmax - 1 can be in the support.  When every row
// of the wave has at most CAPH of them, they are packed into the row's LDS
// scratch crow (by a prefix sum over the row's lanes) and the solve runs on
// CAPH / LPH values per lane instead of NKE.
template <int NKE, int LPH, int CAPH>
__device__ __forceinline__ void threshold_pass(const float* __restrict__ urow, int li, int n,
                                               bool live, int hh, bool smax, float xs_scale,
                                               float ex, int ecls, float* TauX, float* Zs,
                                               float* crow) {
  float xs[NKE];
  float xmax = -INFINITY;
  // U holds kFar past the row's n chunks (up to NKE * LPH), so the values load
  // without a per-entry predicate; all loads are issued before the first use
#pragma unroll
  for (int k = 0; k < NKE; ++k) xs[k] = urow[li + LPH * k];
  __builtin_amdgcn_sched_barrier(0);
#pragma unroll
  for (int k = 0; k < NKE; ++k) {
    xs[k] *= xs_scale;
    xmax = fmaxf(xmax, xs[k]);
  }
  xmax = head_max<LPH>(xmax);
  if (smax) {
    float z = 0.f;
#pragma unroll
    for (int k = 0; k < NKE; ++k) z += exp2f((xs[k] - xmax) * kLog2e);
    z = head_sum<LPH>(z);
    if (live && li == 0) {
      TauX[hh] = xmax;
      Zs[hh] = z;
    }
    return;
  }
  auto solve = [&](const auto& vals, float xout) -> float {
    constexpr int NV = sizeof(vals) / sizeof(float);
    if (ecls == 2) return solve_tau_row<NV, LPH, 2>(vals, xmax, ex, live, xout);
    if (ecls == 1) return solve_tau_row<NV, LPH, 1>(vals, xmax, ex, live, xout);
    if (ecls == 4) return solve_tau_row<NV, LPH, 4>(vals, xmax, ex, live, xout);
    return solve_tau_row<NV, LPH, 0>(vals, xmax, ex, live, xout);
  };
  float tau;
  if constexpr (CAPH / LPH < NKE) {
    const float thr = xmax - 1.f;
    int cnt = 0;
    float xo = -INFINITY;
#pragma unroll
    for (int k = 0; k < NKE; ++k) {
      const bool c = xs[k] > thr;
      cnt += c ? 1 : 0;
      xo = fmaxf(xo, c ? -INFINITY : xs[k]);
    }
    const int incl = head_scan<LPH>(cnt, li);
    const int m = __shfl(incl, (threadIdx.x & 63) | (LPH - 1), 64);  // row total (last lane)
    if (__ballot(live && m > CAPH) == 0ull) {
      int pos = incl - cnt;
#pragma unroll
      for (int k = 0; k < NKE; ++k) {
        if (xs[k] > thr) crow[pos] = xs[k];
        pos += xs[k] > thr ? 1 : 0;
      }
      // the wave reads back what its own lanes wrote (LDS ops of a wave are in order)
      float cv[CAPH / LPH];
#pragma unroll
      for (int j = 0; j < CAPH / LPH; ++j) {
        const int idx = li + LPH * j;
        cv[j] = idx < m ? crow[idx] : kFar;
      }
      tau = solve(cv, head_max<LPH>(xo));
    } else {
      tau = solve(xs, -INFINITY);
    }
  } else {
    tau = solve(xs, -INFINITY);
  }
  if (live && li == 0) TauX[hh] = tau;
}

// Inclusive prefix sum over the 64 lanes of a wave: Hillis-Steele inside each
// 16-lane DPP row (row shifts read 0 past the row's start), then the totals
// of the rows below added from lanes 15, 31 and 47.
template <int S>
__device__ __forceinline__ uint32_t dpp_row_shr(uint32_t v) {
  return (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0x110 + S, 0xF, 0xF, true);
}
__device__ __forceinline__ uint32_t wave_incl_scan(uint32_t v) {
  v += dpp_row_shr<1>(v);
  v += dpp_row_shr<2>(v);
  v += dpp_row_shr<4>(v);
  v += dpp_row_shr<8>(v);
  const uint32_t r0 = (uint32_t)__builtin_amdgcn_readlane((int)v, 15);
  const uint32_t r1 = (uint32_t)__builtin_amdgcn_readlane((int)v, 31);
  const uint32_t r2 = (uint32_t)__builtin_amdgcn_readlane((int)v, 47);
  const int row = (threadIdx.x & 63) >> 4;
  return v + (row >= 1 ? r0 : 0u) + (row >= 2 ? r1 : 0u) + (row >= 3 ? r2 : 0u);
}

// Top-k selection over the n >= 1 non-negative scores S[0..n) (n <= CP; S
// in LDS or global memory): writes the mask words Bits[0 .. ceil(n/64)) with
// exactly kk bits (kk < n) set: every chunk whose score is above the kk-th
// largest, then chunks equal to it in index order.
// The kk-th largest is found by an MSB-first radix select on the scores' bit
// patterns (monotone for non-negative floats), 8 bits a pass, on keys held in
// registers (chunk tid + NTH k in key[k]).  A pass adds its keys to the
// pass's own 256-bin histogram in LDS; wave 0 then scans the bins from the
// top (4 per lane, one wave-wide prefix sum) and publishes the bin of the
// needed key; two barriers a pass.  The passes stop early once that bin holds
// exactly the keys still needed.  Keys equal to the resolved prefix are then
// ranked in index order by one block-wide count.
// hist: 1024 words of LDS; wtot: KPT * NTH / 64 + 3 words.
template <int NTH, int CP>
__device__ __forceinline__ void topk_select(const float* S, int n, int kk, uint64_t* Bits,
                                            uint32_t* hist, int* wtot) {
  constexpr int NW = NTH / 64;
  constexpr int KPT = (CP + NTH - 1) / NTH;
  const int tid = threadIdx.x, lane = tid & 63, wv = tid >> 6;
  int* sel = wtot + KPT * NW;  // digit, keys still needed, keys in its bin
  uint32_t key[KPT];
#pragma unroll
  for (int k = 0; k < KPT; ++k) key[k] = __float_as_uint(S[min(tid + NTH * k, n - 1)]);
  for (int i = tid; i < 1024; i += NTH) hist[i] = 0;
  __syncthreads();
  uint32_t prefix = 0, pmask = 0;
  int need = kk;
  for (int pass = 0; pass < 4; ++pass) {
    const int shift = 24 - 8 * pass;
    uint32_t* hp = hist + 256 * pass;
#pragma unroll
    for (int k = 0; k < KPT; ++k)
      if (tid + NTH * k < n && (key[k] & pmask) == prefix)
        atomicAdd(&hp[(key[k] >> shift) & 255u], 1u);
    __syncthreads();
    if (wv == 0) {
      // lane l holds bins 255-4l (largest) down to 252-4l
      const int top = 255 - 4 * lane;
      const uint32_t h3 = hp[top], h2 = hp[top - 1], h1 = hp[top - 2], h0 = hp[top - 3];
      const uint32_t incl = wave_incl_scan(h0 + h1 + h2 + h3);
      uint32_t a = incl - (h0 + h1 + h2 + h3);  // keys in the bins above this lane's
      const uint32_t nd = (uint32_t)need;
      if (a < nd && nd <= incl) {  // exactly one lane
        int dd;
        uint32_t cnt;
        if (a + h3 >= nd) {
          dd = top; cnt = h3;
        } else if (a + h3 + h2 >= nd) {
          a += h3; dd = top - 1; cnt = h2;
        } else if (a + h3 + h2 + h1 >= nd) {
          a += h3 + h2; dd = top - 2; cnt = h1;
        } else {
          a += h3 + h2 + h1; dd = top - 3; cnt = h0;
        }
        sel[0] = dd;
        sel[1] = (int)(nd - a);
        sel[2] = (int)cnt;
      }
    }
    __syncthreads();
    const int d = sel[0], hd = sel[2];
    need = sel[1];
    prefix |= (uint32_t)d << shift;
    pmask |= 255u << shift;
    if (hd == need) break;  // the whole bin is taken (same on every thread)
  }
  // every key above the prefix on the resolved bits, and the first `need`
  // keys equal to it there
  uint64_t eqm[KPT];
#pragma unroll
  for (int k = 0; k < KPT; ++k) {
    const bool eq = tid + NTH * k < n && (key[k] & pmask) == prefix;
    eqm[k] = __ballot(eq);
    if (lane == 0) wtot[k * NW + wv] = __popcll(eqm[k]);
  }
  __syncthreads();
  int before = 0;  // equal keys in the blocks k' < k
#pragma unroll
  for (int k = 0; k < KPT; ++k) {
    const int c = tid + NTH * k;
    int pre = 0, all = 0;
#pragma unroll
    for (int w = 0; w < NW; ++w) {
      const int t = wtot[k * NW + w];
      pre += w < wv ? t : 0;
      all += t;
    }
    const uint32_t km = key[k] & pmask;
    const bool eq = (eqm[k] >> lane) & 1ull;
    const int rank = before + pre + (int)__popcll(eqm[k] & ((1ull << lane) - 1ull));
    const bool on = c < n && (km > prefix || (eq && rank < need));
    const uint64_t b = __ballot(on);
    const int word = k * NW + wv;
    if (lane == 0 && word < (n + 63) / 64) Bits[word] = b;
    before += all;
  }
}

// NTH = 256 (prefill: many rows) or 1024 (decode: one workgroup per
// sequence and KV head, so 16 waves share the logits and one wave solves each
// query head's threshold).
template <bool BF16, int D, int CP, int NTH>
__device__ __forceinline__ void route_row(const Geom& g, const RouteParams& p, int64_t row, int h) {
  constexpr int NW = NTH / 64;              // waves
  constexpr int LPH = NW == 16 ? 64 : (CP > 1024 ? 32 : 16);  // lanes per head in the solve
  constexpr int HPW = 64 / LPH;             // heads per wave per pass
  constexpr int NK = CP / LPH;              // values per lane in the solve
  constexpr int USTR = CP + 16;     // LDS row stride: rows start 16 banks apart
  constexpr int CAPH = LPH == 64 ? 256 : 8 * LPH;  // packed candidates per head row
  __shared__ float U[16 * USTR];    // logits of one 16-head tile
  __shared__ float Cand[16 * CAPH]; // packed threshold candidates, per head row
  __shared__ float Wsum[CP];        // sum over the group's heads of p
  __shared__ uint64_t Bits[CP / 64];
  __shared__ float TauX[16];        // threshold (x units), or max u (softmax)
  __shared__ float Zs[16];          // softmax denominator (alpha = 1)
  __shared__ int Wtot[((CP + NTH - 1) / NTH) * NW + 3];  // top-k: equal keys per wave

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
    for (int w = tid; w < g.W; w += NTH) mrow[w] = 0ull;
    if (p.tau)
      for (int q = tid; q < g.G; q += NTH)
        p.tau[(int64_t)(h * g.G + q) * rows + tok] = INFINITY;
    return;
  }
  // entries of each head's entmax: the routed chunks, then the estimated
  // summary of the row's own chunk when given (column n of U)
  const int ns = p.kdiag ? n + 1 : n;
  const uint16_t* kdrow = (const uint16_t*)p.kdiag + ((tok * g.Hkv + h) * (int64_t)D) * (BF16 ? 1 : 2);
  // top-k routing scores chunks by the group's summed softmax probabilities
  const bool topk = p.topk > 0;
  if (topk) alpha = 1.f;
  const bool smax = !(alpha > 1.f);
  const float am1 = alpha - 1.f;
  const float ex = smax ? 1.f : 1.f / am1;
  const int ecls = smax ? 0 : (ex == 1.f ? 1 : (ex == 2.f ? 2 : (ex == 4.f ? 4 : 0)));
  const float xs_scale = smax ? 1.f : am1;

  for (int c = tid; c < n; c += NTH) Wsum[c] = 0.f;
  for (int w = tid; w < CP / 64; w += NTH) Bits[w] = 0ull;

  const int ntile_h = (g.G + 15) / 16;
  for (int ht = 0; ht < ntile_h; ++ht) {
    const int h0 = ht * 16;
    const int nh = min(16, g.G - h0);
    __syncthreads();
    // ---- 1. logits U[q][c]: 16 heads x 16 chunks per MFMA tile, the
    //         summary loads of 4 tiles issued before their MFMAs
    if constexpr (BF16) {
      constexpr int KS = D / 32;
      const int r = lane & 15, gq = lane >> 4;
      bf16x8 qa[KS];
      const uint16_t* qrow =
          (const uint16_t*)p.q + ((tok * g.Hq + h * g.G + h0 + r) * (int64_t)D);
#pragma unroll
      for (int ks = 0; ks < KS; ++ks) {
        u32x4 v = {0u, 0u, 0u, 0u};
        if (r < nh) v = ldg16(qrow + 32 * ks + 8 * gq);
        qa[ks] = as_bf16x8(v);
      }
      const int nct = (ns + 15) >> 4;
      for (int ct0 = 4 * wv; ct0 < nct; ct0 += 4 * NW) {
        u32x4 kv[4][KS];
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          // clamped to a valid entry; columns past ns are discarded below
          const int c = min((ct0 + j) * 16 + r, ns - 1);
          const uint16_t* krow =
              c == n ? kdrow : (const uint16_t*)p.kbar + (((kb0 + c) * g.Hkv + h) * (int64_t)D);
#pragma unroll
          for (int ks = 0; ks < KS; ++ks) kv[j][ks] = ldg16(krow + 32 * ks + 8 * gq);
        }
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          const int c = (ct0 + j) * 16 + r;
          f32x4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
          for (int ks = 0; ks < KS; ++ks) acc = mfma16x16x32(qa[ks], as_bf16x8(kv[j][ks]), acc);
          if (c < ns) {
#pragma unroll
            for (int jj = 0; jj < 4; ++jj) U[(4 * gq + jj) * USTR + c] = acc[jj] * p.gamma_scale;
          }
        }
      }
    } else {
      for (int idx = tid; idx < nh * ns; idx += NTH) {
        const int hh = idx / ns, c = idx - hh * ns;
        const float* qr = (const float*)p.q + ((tok * g.Hq + h * g.G + h0 + hh) * (int64_t)D);
        const float* kr = c == n ? (const float*)kdrow
                                 : (const float*)p.kbar + (((kb0 + c) * g.Hkv + h) * (int64_t)D);
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
        U[hh * USTR + c] = d * p.gamma_scale;
      }
    }
    // entries from ns up to the row's solve width hold a sentinel far below any
    // threshold (kFar / xs_scale stays far below after scaling)
    {
      const int npad = ns <= (NK / 4) * LPH && NK >= 16 ? (NK / 4) * LPH
                       : ns <= (NK / 2) * LPH && NK >= 8 ? (NK / 2) * LPH : CP;
      const int w = npad - ns;
      for (int idx = tid; idx < 16 * w; idx += NTH) {
        const int hh = idx / w;
        U[hh * USTR + ns + (idx - hh * w)] = kFar;
      }
    }
    __syncthreads();
    // ---- 2. thresholds: each pass gives every wave HPW heads, LPH lanes each
    for (int hb = 0; hb < nh; hb += NW * HPW) {
      const int hh = hb + wv * HPW + lane / LPH;
      const int li = lane % LPH;
      const bool live = hh < nh;
      const float* urow = U + (hh & 15) * USTR;  // in bounds for every lane
      float* crow = Cand + (hh & 15) * CAPH;
      // values per lane for this row's ns entries: a quarter, half or all of NK
      if (ns <= (NK / 4) * LPH && NK >= 16)
        threshold_pass<(NK >= 16 ? NK / 4 : NK), LPH, CAPH>(urow, li, ns, live, hh, smax, xs_scale,
                                                            ex, ecls, TauX, Zs, crow);
      else if (ns <= (NK / 2) * LPH && NK >= 8)
        threshold_pass<(NK >= 8 ? NK / 2 : NK), LPH, CAPH>(urow, li, ns, live, hh, smax, xs_scale,
                                                           ex, ecls, TauX, Zs, crow);
      else
        threshold_pass<NK, LPH, CAPH>(urow, li, ns, live, hh, smax, xs_scale, ex, ecls, TauX, Zs,
                                      crow);
    }
    __syncthreads();
    if (p.tau && tid < nh)
      p.tau[(int64_t)(h * g.G + h0 + tid) * rows + tok] =
          topk ? NAN : (smax ? -INFINITY : TauX[tid] / am1);
    // ---- 3. group weight numerators and active bits
    // (the exponent's form fixed at compile time, the 16 rows of the tile read
    // unconditionally and rows past nh masked by selects: no branch per entry,
    // all LDS reads of a chunk in flight together)
    auto weights = [&](auto ecls_tag) {
      constexpr int E = decltype(ecls_tag)::value;
      float tx[16], zi[16];
#pragma unroll
      for (int hh = 0; hh < 16; ++hh) {
        tx[hh] = TauX[hh];
        zi[hh] = E < 0 ? 1.f / Zs[hh] : 0.f;
      }
      for (int base = 0; base < n; base += NTH) {
        const int c = base + tid;
        const int cc = min(c, n - 1);
        float uu[16];
#pragma unroll
        for (int hh = 0; hh < 16; ++hh) uu[hh] = U[hh * USTR + cc];
        __builtin_amdgcn_sched_barrier(0);
        bool on = false;
        float w0 = 0.f, w1 = 0.f;
#pragma unroll
        for (int hh = 0; hh < 16; ++hh) {
          const bool valid = hh < nh;
          float v;
          if constexpr (E < 0) {
            v = exp2f((uu[hh] - tx[hh]) * kLog2e) * zi[hh];
            on = on || valid;
          } else {
            const float d = uu[hh] * am1 - tx[hh];
            on = on || (valid && d > 0.f);
            float pd;
            pow_pair<E>(fmaxf(d, 0.f), ex, v, pd);
          }
          v = valid ? v : 0.f;
          if (hh & 1) w1 += v; else w0 += v;
        }
        on = on && c < n;
        if (c < n) Wsum[c] += w0 + w1;
        const uint64_t b = __ballot(on);
        if (lane == 0 && (base >> 6) + wv < CP / 64) Bits[(base >> 6) + wv] |= b;
      }
    };
    if (smax) weights(std::integral_constant<int, -1>());
    else if (ecls == 2) weights(std::integral_constant<int, 2>());
    else if (ecls == 1) weights(std::integral_constant<int, 1>());
    else if (ecls == 4) weights(std::integral_constant<int, 4>());
    else weights(std::integral_constant<int, 0>());
  }
  __syncthreads();
  if (topk && p.topk < n) {
    // the candidate scratch (free by now) holds the radix histograms
    static_assert(16 * CAPH >= 1024, "histogram space");
    topk_select<NTH, CP>(Wsum, n, p.topk, Bits, reinterpret_cast<uint32_t*>(Cand), Wtot);
    __syncthreads();
  }
  if (p.log_prior) {
    float* lrow = p.log_prior + ((int64_t)h * rows + tok) * g.C_slots;
    const float invG = 1.f / (float)g.G;
    for (int c = tid; c < n; c += NTH) {
      const bool on = (Bits[c >> 6] >> (c & 63)) & 1ull;
      float v = -INFINITY;
      if (on)
        v = (topk || p.sigma == 0.f) ? 0.f : p.sigma * logf(fmaxf(Wsum[c] * invG, 1e-38f));
      lrow[c] = v;
    }
  }
  for (int w = tid; w < g.W; w += NTH) mrow[w] = (w < CP / 64) ? Bits[w] : 0ull;
}

template <bool BF16, int D, int CP, int NTH>
__global__ __launch_bounds__(NTH) void route_kernel(Geom g, RouteParams p) {
  route_row<BF16, D, CP, NTH>(g, p, p.row0 + blockIdx.x, blockIdx.y);
}

// The rows the streaming routing flagged (a head's candidate list outgrew
// its capacity, or softmax routing), routed again one workgroup per row with
// the whole logit row in LDS.  Every workgroup of KV head blockIdx.y counts
// the head's flagged rows (thread t reads the flag words t, t + 256, ...,
// four rows a word) and takes those of rank blockIdx.x, blockIdx.x +
// gridDim.x, ... in that order: the flagged rows spread evenly over the grid
// however they cluster, and a workgroup with none of them is done after one
// read of the flags.
template <int D, int CP>
__global__ __launch_bounds__(256) void route_fallback_kernel(Geom g, RouteParams p,
                                                             const uint8_t* __restrict__ flags) {
  __shared__ int wsum[4];
  __shared__ int64_t pick;
  const int tid = threadIdx.x, lane = tid & 63, wv = tid >> 6;
  const int h = blockIdx.y;
  const uint32_t* fw = (const uint32_t*)(flags + (int64_t)h * route_flag_stride(p.rows));
  const int64_t nw = (p.rows + 3) / 4;
  // word w's flags (one byte per row, 0 or 1), bytes past the last row cleared
  auto word = [&](int64_t w) -> uint32_t {
    const int64_t left = p.rows - 4 * w;
    return fw[w] & (left >= 4 ? 0xffffffffu : (1u << (8 * left)) - 1u);
  };
  int cnt = 0;
  for (int64_t w = tid; w < nw; w += 256) cnt += __popc(word(w));
  int inc = cnt;
#pragma unroll
  for (int o = 1; o < 64; o <<= 1) {
    const int y = __shfl_up(inc, o);
    if (lane >= o) inc += y;
  }
  if (lane == 63) wsum[wv] = inc;
  __syncthreads();
  int before = 0, total = 0;
#pragma unroll
  for (int w = 0; w < 4; ++w) {
    before += w < wv ? wsum[w] : 0;
    total += wsum[w];
  }
  const int base = before + inc - cnt;  // rank of this thread's first flagged row
  for (int k = blockIdx.x; k < total; k += gridDim.x) {
    if (k >= base && k < base + cnt) {
      int want = k - base;
      for (int64_t w = tid; w < nw; w += 256) {
        uint32_t v = word(w);
        const int c = __popc(v);
        if (want < c) {
          for (; want > 0; --want) v &= v - 1;
          pick = 4 * w + (__ffs(v) - 1) / 8;
          break;
        }
        want -= c;
      }
    }
    __syncthreads();
    const int64_t row = pick;
    __syncthreads();
    route_row<true, D, CP, 256>(g, p, row, h);
  }
}

// Routing logits for a few rows (decode): u[q][c] = gamma*s*<q, k_bar_c> for
// every routable chunk of each row, 16 heads x 16 chunks per MFMA tile (bf16,
// fp32 accumulate), one tile per wave and 64 chunks per workgroup, so that the
// summary reads spread over the whole chip instead of one CU per row.  Written
// to the scratch [rows, Hkv, G, C_slots] that the solve and weight passes read.
// With p.app_knew, one more workgroup per (row, KV head), the last of its grid
// row, appends the row's new token to the caches (append_token), fused into
// the step.
template <int D>
__global__ __launch_bounds__(256) void route_logits_kernel(Geom g, RouteParams p) {
  constexpr int KS = D / 32;
  const int tid = threadIdx.x, lane = tid & 63, wv = tid >> 6;
  const int r = lane & 15, gq = lane >> 4;
  const int row = blockIdx.y, h = blockIdx.z;
  if (p.app_knew && blockIdx.x == gridDim.x - 1) {  // the fused append's column
    if (tid < kWave)
      append_token<true, D>(g, p.app_knew, p.app_vnew, p.seqlens, p.app_qbar, p.app_kc,
                            p.app_vc, p.app_kbar, row, h);
    return;
  }
  const int n = (p.seqlens[row] - 1) / g.B;
  // entries: the routed chunks, then the row's own-chunk estimate when given
  const int ns = (p.kdiag && n > 0) ? n + 1 : n;
  const int c0 = (blockIdx.x * 4 + wv) * 16;  // this wave's 16 chunks
  if (c0 >= ns) return;
  const int64_t kb0 = (int64_t)row * (g.max_seqlen / g.B);
  // clamped to a valid entry; columns past ns are not written
  const int c = min(c0 + r, ns - 1);
  const uint16_t* krow =
      c == n ? (const uint16_t*)p.kdiag + (((int64_t)row * g.Hkv + h) * D)
             : (const uint16_t*)p.kbar + (((kb0 + c) * g.Hkv + h) * (int64_t)D);
  u32x4 kv[KS];
#pragma unroll
  for (int ks = 0; ks < KS; ++ks) kv[ks] = ldg16(krow + 32 * ks + 8 * gq);
  for (int h0 = 0; h0 < g.G; h0 += 16) {
    const int nh = min(16, g.G - h0);
    const uint16_t* qrow =
        (const uint16_t*)p.q + (((int64_t)row * g.Hq + h * g.G + h0 + r) * D);
    f32x4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) {
      u32x4 v = {0u, 0u, 0u, 0u};
      if (r < nh) v = ldg16(qrow + 32 * ks + 8 * gq);
      acc = mfma16x16x32(as_bf16x8(v), as_bf16x8(kv[ks]), acc);
    }
    // lane (gq, r): heads 4 gq + j, chunk c0 + r
    if (c0 + r < ns) {
      float* ur = p.ulog + (((int64_t)row * g.Hkv + h) * g.G + h0) * g.C_slots + c0 + r;
#pragma unroll
      for (int j = 0; j < 4; ++j)
        if (4 * gq + j < nh) ur[(int64_t)(4 * gq + j) * g.C_slots] = acc[j] * p.gamma_scale;
    }
  }
}

// Threshold of one decode row held by a wave (xs[k]: entry li + 64 k), on a
// short candidate list.  The entmax root of the 64 lane maxima is a lower
// bound b on tau (a subset of the entries has no more mass at any threshold,
// so its root is no larger); a few Newton steps from below reach it, less a
// relative rounding margin.  Only entries above b can be in the support, and
// on these inputs they are about as many as the support itself (tens of the
// 2048); they are compacted into LDS and the threshold solved on them alone,
// NKC values a lane instead of NK.  A longer list solves on the whole row.
constexpr int kDecBoundIters = 6;
template <int NK, int NKC, int ECLS>
__device__ float solve_tau_compact(const float (&xs)[NK], float xmax, float ex, float* cand) {
  const int li = threadIdx.x & 63;
  float lm = -INFINITY;
#pragma unroll
  for (int k = 0; k < NK; ++k) lm = fmaxf(lm, xs[k]);
  float b = xmax - 1.f;  // the top entry alone has mass 1 here
#pragma unroll
  for (int it = 0; it < kDecBoundIters; ++it) {
    float pw, pd;
    pow_pair<ECLS>(fmaxf(lm - b, 0.f), ex, pw, pd);
    const float f = head_sum<64>(pw), fd = head_sum<64>(pd);
    const float step = (f - 1.f) / (ex * fd);
    b = (step > 0.f && fd > 0.f) ? b + step : b;
  }
  b -= 1e-4f * fmaxf(1.f, fabsf(b));
  int cnt = 0;
  float xo = -INFINITY;
#pragma unroll
  for (int k = 0; k < NK; ++k) {
    const bool c = xs[k] > b;
    cnt += c ? 1 : 0;
    xo = fmaxf(xo, c ? -INFINITY : xs[k]);
  }
  const int incl = head_scan<64>(cnt, li);
  const int m = __shfl(incl, 63, 64);  // list length (last lane's inclusive count)
  if (m > 64 * NKC) return solve_tau_row<NK, 64, ECLS>(xs, xmax, ex, true, -INFINITY);
  int pos = incl - cnt;
#pragma unroll
  for (int k = 0; k < NK; ++k) {
    if (xs[k] > b) cand[pos] = xs[k];
    pos += xs[k] > b ? 1 : 0;
  }
  // the wave reads back what its own lanes wrote (LDS ops of a wave are in order)
  float cv[NKC];
#pragma unroll
  for (int j = 0; j < NKC; ++j) cv[j] = li + 64 * j < m ? cand[li + 64 * j] : kFar;
  return solve_tau_row<NKC, 64, ECLS>(cv, xmax, ex, true, head_max<64>(xo));
}

// Decode threshold solve: one wave per (query head, row, KV head) reads the
// head's logits row from the scratch (CP / 64 values per lane) and writes its
// threshold in x units (alpha > 1), or its maximum and softmax denominator
// (alpha = 1), to tsx[row, Hkv, G, 2]; tau (u units) if requested.
template <int CP>
__global__ __launch_bounds__(64) void route_solve_kernel(Geom g, RouteParams p) {
  constexpr int NK = CP / 64;
  const int q = blockIdx.x, row = blockIdx.y, h = blockIdx.z;
  const int li = threadIdx.x;
  const int64_t rows = p.rows;
  const int n = (p.seqlens[row] - 1) / g.B;
  float* ts = p.tsx + (((int64_t)row * g.Hkv + h) * g.G + q) * 2;
  if (n <= 0) {
    if (li == 0 && p.tau) p.tau[(int64_t)(h * g.G + q) * rows + row] = INFINITY;
    return;
  }
  const float alpha = p.alpha;
  const bool smax = !(alpha > 1.f);
  const float am1 = alpha - 1.f;
  const float ex = smax ? 1.f : 1.f / am1;
  const int ecls = smax ? 0 : (ex == 1.f ? 1 : (ex == 2.f ? 2 : (ex == 4.f ? 4 : 0)));
  const float xs_scale = smax ? 1.f : am1;
  const float* ur = p.ulog + (((int64_t)row * g.Hkv + h) * g.G + q) * g.C_slots;
  // entries: the routed chunks, then the own-chunk estimate when given
  const int ns = p.kdiag ? n + 1 : n;
  // every load unconditional (clamped to the row) and in flight together;
  // entries past ns become the sentinel afterwards
  float xs[NK];
#pragma unroll
  for (int k = 0; k < NK; ++k) xs[k] = ur[min(li + 64 * k, ns - 1)];
  __builtin_amdgcn_sched_barrier(0);
#pragma unroll
  for (int k = 0; k < NK; ++k) xs[k] = li + 64 * k < ns ? xs[k] * xs_scale : kFar;
  float xmax = -INFINITY;
#pragma unroll
  for (int k = 0; k < NK; ++k) xmax = fmaxf(xmax, xs[k]);
  xmax = head_max<64>(xmax);
  if (smax) {
    float z = 0.f;
#pragma unroll
    for (int k = 0; k < NK; ++k) z += exp2f((xs[k] - xmax) * kLog2e);
    z = head_sum<64>(z);
    if (li == 0) {
      ts[0] = xmax;
      ts[1] = z;
      if (p.tau) p.tau[(int64_t)(h * g.G + q) * rows + row] = -INFINITY;
    }
    return;
  }
  __shared__ float cand[128];
  constexpr int NKC = NK < 2 ? NK : 2;
  float tau;
  if (ecls == 2) tau = solve_tau_compact<NK, NKC, 2>(xs, xmax, ex, cand);
  else if (ecls == 1) tau = solve_tau_compact<NK, NKC, 1>(xs, xmax, ex, cand);
  else if (ecls == 4) tau = solve_tau_compact<NK, NKC, 4>(xs, xmax, ex, cand);
  else tau = solve_tau_compact<NK, NKC, 0>(xs, xmax, ex, cand);
  if (li == 0) {
    ts[0] = tau;
    ts[1] = 0.f;
    if (p.tau) p.tau[(int64_t)(h * g.G + q) * rows + row] = tau / am1;
  }
}

// Decode group weights: one thread per routable chunk c of a (row, KV head):
// w_bar_c = (1/G) sum_q [x_qc - tau_q]_+^(1/(alpha-1)) (softmax: the mean of
// the heads' softmax probabilities), the active bit OR_q [x_qc > tau_q]
// gathered 64 chunks per wave into one mask word, and the log-prior
// sigma*log(w_bar_c) on the active chunks.
template <int E>
__global__ __launch_bounds__(256) void route_weights_kernel(Geom g, RouteParams p) {
  const int tid = threadIdx.x, lane = tid & 63, wv = tid >> 6;
  const int row = blockIdx.y, h = blockIdx.z;
  const int64_t rows = p.rows;
  const int c = blockIdx.x * 256 + tid;
  const int word = blockIdx.x * 4 + wv;
  if (word * 64 >= g.C_slots) return;
  const int n = (p.seqlens[row] - 1) / g.B;
  const float am1 = p.alpha - 1.f;
  const float ex = E < 0 ? 1.f : 1.f / am1;
  const float* ts = p.tsx + ((int64_t)row * g.Hkv + h) * g.G * 2;
  const float* ur = p.ulog + ((int64_t)row * g.Hkv + h) * g.G * g.C_slots;
  bool on = false;
  float w = 0.f;
  // 16 heads at a time, every load unconditional (clamped) and in flight
  // together; heads past G and chunks past n are masked by selects
  const int cc = min(c, max(n - 1, 0));
  for (int q0 = 0; q0 < g.G; q0 += 16) {
    float uu[16], t0[16], t1[16];
#pragma unroll
    for (int j = 0; j < 16; ++j) {
      const int q = min(q0 + j, g.G - 1);
      uu[j] = ur[(int64_t)q * g.C_slots + cc];
      t0[j] = ts[2 * q];
      t1[j] = ts[2 * q + 1];
    }
    __builtin_amdgcn_sched_barrier(0);
#pragma unroll
    for (int j = 0; j < 16; ++j) {
      const bool valid = q0 + j < g.G && c < n;
      float v;
      if constexpr (E < 0) {
        v = exp2f((uu[j] - t0[j]) * kLog2e) / t1[j];
        on = on || valid;
      } else {
        const float d = uu[j] * am1 - t0[j];
        on = on || (valid && d > 0.f);
        float pd;
        pow_pair<E>(fmaxf(d, 0.f), ex, v, pd);
      }
      w += valid ? v : 0.f;
    }
  }
  if (p.topk > 0) {  // top-k: the group score, selected by the next pass
    if (c < n) p.score[((int64_t)row * g.Hkv + h) * g.C_slots + c] = w;
    return;
  }
  const uint64_t bits = __ballot(on);
  if (lane == 0) p.mask[((int64_t)h * rows + row) * g.W + word] = bits;
  if (p.log_prior && c < g.C_slots) {
    float v = -INFINITY;
    if (on) v = (p.sigma == 0.f) ? 0.f : p.sigma * logf(fmaxf(w / (float)g.G, 1e-38f));
    p.log_prior[((int64_t)h * rows + row) * g.C_slots + c] = v;
  }
}

// Decode top-k selection: one 4-wave workgroup per (row, KV head) keeps the
// min(k, n) largest group scores of the row (ties to the lower chunk index),
// read straight from the scratch, and writes the mask words and the
// log-prior (0 on the kept chunks, -inf on the other routable ones).
template <int CP>
__global__ __launch_bounds__(256) void route_topk_select_kernel(Geom g, RouteParams p) {
  constexpr int NTH = 256;
  __shared__ uint64_t Bits[CP / 64];
  constexpr int KPT = (CP + NTH - 1) / NTH;
  __shared__ uint32_t Hist[1024];
  __shared__ int Wtot[KPT * (NTH / 64) + 3];
  const int row = blockIdx.x, h = blockIdx.y;
  const int tid = threadIdx.x;
  const int64_t rows = p.rows;
  const int n = (p.seqlens[row] - 1) / g.B;
  uint64_t* mrow = p.mask + ((int64_t)h * rows + row) * g.W;
  if (n <= 0) {
    for (int w = tid; w < g.W; w += NTH) mrow[w] = 0ull;
    return;
  }
  // every routable chunk when k >= n; the selection overwrites words < ceil(n/64)
  for (int w = tid; w < CP / 64; w += NTH) {
    const int lo = 64 * w;
    Bits[w] = lo + 64 <= n ? ~0ull : (lo < n ? (1ull << (n - lo)) - 1ull : 0ull);
  }
  if (p.topk < n)
    topk_select<NTH, CP>(p.score + ((int64_t)row * g.Hkv + h) * g.C_slots, n, p.topk, Bits,
                         Hist, Wtot);
  __syncthreads();
  if (p.log_prior) {
    float* lrow = p.log_prior + ((int64_t)h * rows + row) * g.C_slots;
    uint64_t wd[KPT];
#pragma unroll
    for (int k = 0; k < KPT; ++k) wd[k] = Bits[min((tid + NTH * k) >> 6, CP / 64 - 1)];
#pragma unroll
    for (int k = 0; k < KPT; ++k) {
      const int c = tid + NTH * k;
      if (c < n) lrow[c] = ((wd[k] >> (c & 63)) & 1ull) ? 0.f : -INFINITY;
    }
  }
  for (int w = tid; w < g.W; w += NTH) mrow[w] = (w < CP / 64) ? Bits[w] : 0ull;
}

hipError_t launch_route_fallback(const Geom& g, const RouteParams& p, const uint8_t* flags,
                                 hipStream_t st) {
  dim3 grid((unsigned)std::min<int64_t>(p.rows, 256), g.Hkv);
#define DASH_FB(DD, CPV) \
  hipLaunchKernelGGL((route_fallback_kernel<DD, CPV>), grid, dim3(256), 0, st, g, p, flags)
#define DASH_FB_CP(DD)                                 \
  do {                                                 \
    if (g.C_slots <= 256) DASH_FB(DD, 256);            \
    else if (g.C_slots <= 512) DASH_FB(DD, 512);       \
    else if (g.C_slots <= 1024) DASH_FB(DD, 1024);     \
    else DASH_FB(DD, 2048);                            \
  } while (0)
  if (g.D == 64) DASH_FB_CP(64); else DASH_FB_CP(128);
#undef DASH_FB_CP
#undef DASH_FB
  return hipGetLastError();
}

hipError_t launch_route(const Geom& g, const RouteParams& p, hipStream_t st) {
  if (p.rows == 0) return hipSuccess;
  dim3 grid((unsigned)p.rows, g.Hkv);
  // few rows (decode, bf16): logits, per-head thresholds and per-chunk
  // weights as three chip-wide passes through the scratch; few rows in fp32:
  // one 16-wave workgroup per row; many rows (prefill): 4 waves per row
  const bool wide = p.seqlens != nullptr;
  if (wide && g.bf16 && p.ulog != nullptr && p.tsx != nullptr &&
      (p.topk <= 0 || p.score != nullptr)) {
    dim3 lgrid((unsigned)((g.C_slots + 63) / 64 + (p.app_knew ? 1 : 0)), (unsigned)p.rows, g.Hkv);
    if (g.D == 64) hipLaunchKernelGGL(route_logits_kernel<64>, lgrid, dim3(256), 0, st, g, p);
    else hipLaunchKernelGGL(route_logits_kernel<128>, lgrid, dim3(256), 0, st, g, p);
    dim3 sgrid(g.G, (unsigned)p.rows, g.Hkv);
    if (g.C_slots <= 256) hipLaunchKernelGGL(route_solve_kernel<256>, sgrid, dim3(64), 0, st, g, p);
    else if (g.C_slots <= 512) hipLaunchKernelGGL(route_solve_kernel<512>, sgrid, dim3(64), 0, st, g, p);
    else if (g.C_slots <= 1024) hipLaunchKernelGGL(route_solve_kernel<1024>, sgrid, dim3(64), 0, st, g, p);
    else hipLaunchKernelGGL(route_solve_kernel<2048>, sgrid, dim3(64), 0, st, g, p);
    dim3 wgrid((unsigned)((g.C_slots + 255) / 256), (unsigned)p.rows, g.Hkv);
    const float am1 = p.alpha - 1.f;
    const float ex = am1 > 0.f ? 1.f / am1 : 1.f;
    if (!(p.alpha > 1.f)) hipLaunchKernelGGL(route_weights_kernel<-1>, wgrid, dim3(256), 0, st, g, p);
    else if (ex == 2.f) hipLaunchKernelGGL(route_weights_kernel<2>, wgrid, dim3(256), 0, st, g, p);
    else if (ex == 1.f) hipLaunchKernelGGL(route_weights_kernel<1>, wgrid, dim3(256), 0, st, g, p);
    else if (ex == 4.f) hipLaunchKernelGGL(route_weights_kernel<4>, wgrid, dim3(256), 0, st, g, p);
    else hipLaunchKernelGGL(route_weights_kernel<0>, wgrid, dim3(256), 0, st, g, p);
    if (p.topk > 0) {
      dim3 tgrid((unsigned)p.rows, g.Hkv);
      if (g.C_slots <= 256) hipLaunchKernelGGL(route_topk_select_kernel<256>, tgrid, dim3(256), 0, st, g, p);
      else if (g.C_slots <= 512) hipLaunchKernelGGL(route_topk_select_kernel<512>, tgrid, dim3(256), 0, st, g, p);
      else if (g.C_slots <= 1024) hipLaunchKernelGGL(route_topk_select_kernel<1024>, tgrid, dim3(256), 0, st, g, p);
      else hipLaunchKernelGGL(route_topk_select_kernel<2048>, tgrid, dim3(256), 0, st, g, p);
    }
    return hipGetLastError();
  }
#define DASH_ROUTE(BF, DD, CPV)                                                                \
  do {                                                                                         \
    if (wide)                                                                                  \
      hipLaunchKernelGGL((route_kernel<BF, DD, CPV, 1024>), grid, dim3(1024), 0, st, g, p);        \
    else                                                                                       \
      hipLaunchKernelGGL((route_kernel<BF, DD, CPV, 256>), grid, dim3(256), 0, st, g, p);          \
  } while (0)
#define DASH_ROUTE_CP(BF, DD)                                                     \
  do {                                                                            \
    if (g.C_slots <= 256) DASH_ROUTE(BF, DD, 256);                                \
    else if (g.C_slots <= 512) DASH_ROUTE(BF, DD, 512);                           \
    else if (g.C_slots <= 1024) DASH_ROUTE(BF, DD, 1024);                         \
    else DASH_ROUTE(BF, DD, 2048);                                                \
  } while (0)
  if (!wide && !g.cu_seqlens && g.num_seqs == 1 && p.rows == g.T && p.row0 == 0 &&
      g.C_slots > 256) {
    // one sequence: a row at position i has floor(i/B) routable chunks, so the
    // rows below CP*B fit the CP-wide variant (less LDS, a shorter candidate
    // scan); each range runs its own variant, the longest rows first
    for (int cp = 2048; cp >= 256; cp /= 2) {
      if (cp > 256 && (int64_t)(cp / 2) >= g.C_slots) continue;
      const int64_t hi = std::min<int64_t>(p.rows, (int64_t)cp * g.B);
      const int64_t lo = cp == 256 ? 0 : std::min<int64_t>(p.rows, (int64_t)(cp / 2) * g.B);
      if (hi <= lo) continue;
      RouteParams q = p;
      q.row0 = lo;
      dim3 rgrid((unsigned)(hi - lo), g.Hkv);
#define DASH_RANGE(BF, DD, CPV) \
  hipLaunchKernelGGL((route_kernel<BF, DD, CPV, 256>), rgrid, dim3(256), 0, st, g, q)
#define DASH_RANGE_CP(BF, DD)                   \
  do {                                          \
    if (cp == 256) DASH_RANGE(BF, DD, 256);     \
    else if (cp == 512) DASH_RANGE(BF, DD, 512); \
    else if (cp == 1024) DASH_RANGE(BF, DD, 1024); \
    else DASH_RANGE(BF, DD, 2048);              \
  } while (0)
      if (g.bf16) {
        if (g.D == 64) DASH_RANGE_CP(true, 64); else DASH_RANGE_CP(true, 128);
      } else {
        if (g.D == 64) DASH_RANGE_CP(false, 64); else DASH_RANGE_CP(false, 128);
      }
#undef DASH_RANGE_CP
#undef DASH_RANGE
    }
    return hipGetLastError();
  }
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
