// Phase 1 for many prefill rows, streaming ("Fase 1: Entmax Chunk Routering"
// of the gist.science technical summary: w_hat = alpha-entmax(gamma z_bar) per
// query head, the heads of a GQA group averaged into one shared support).
//
// One workgroup of four waves routes R = 4 * RPW consecutive positions of one
// sequence against one KV head's summaries; each wave owns RPW rows and all
// G = 16 * HT query heads of its KV head.  No row of logits is kept: the
// logits u = gamma * s * <q, k_bar> (16 heads x 16 chunks per bf16 MFMA tile,
// fp32 accumulate, the summaries read straight from global memory three tiles
// ahead) are recomputed in three passes over the chunks, and in x = (alpha-1) u:
//   1. each lane keeps, per (row, head), the largest x of the chunks it
//      holds (chunk 16 t + lane % 16): 16 partial maxima per (row, head).
//      The entmax mass f(t) = sum_c [x_c - t]_+^(1/(alpha-1)) taken over
//      those 16 values alone is at most the full mass, so its root (a few
//      Newton steps from below, started at max - 1 where the top value alone
//      has mass 1) is a lower bound b <= tau;
//   2. every x > b of the row and head (a superset of the support, about
//      the support's size) is appended to the head's candidate list in LDS;
//   3. tau from the candidates alone (Newton from b, then the sort-free
//      closed form of alpha = 2 and alpha = 1.5 on the support found); the
//      third pass forms, per chunk, p_qc = [x_qc - tau_q]_+^(1/(alpha-1)),
//      w_bar_c = mean over the G heads, the active bit w_bar_c > 0
//      and the log-prior sigma * log(w_bar_c), and writes the mask words and
//      the prior row directly.
// A row with a head whose candidates outgrow the list (nearly uniform
// logits) is flagged instead; route_fallback_kernel then routes the flagged
// rows again with whole logit rows in LDS.  Every row's flag is written, 0
// or 1, on every call.
#include "dash_device.h"
#include "dash_internal.h"

namespace dash {

constexpr int kRrWaves = 4;
constexpr int kRrCap = 64;     // candidates per (row, head)
constexpr int kRrBoundIters = 4;

// d^e and d^(e-1) for d >= 0: e = 1, 2, 4 exactly (ECLS), else through
// exp2(e log2 d), which is 0 at d = 0.
template <int ECLS>
__device__ __forceinline__ void rr_pow(float d, float e, float& pw, float& pd) {
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
    pw = d > 0.f ? exp2f(e * lg) : 0.f;
    pd = d > 0.f ? exp2f((e - 1.f) * lg) : 0.f;
  }
}

// LDS of one workgroup.  A candidate list row is padded by one word so that
// the 64 lanes reading their own lists hit 64 different banks.
struct RrShared {
  float cand[kRrWaves][64][kRrCap + 1];
  int cnt[kRrWaves][64];
  float bnd[kRrWaves][64];
  float tau[kRrWaves][64];
};
constexpr int kRrAhead = 3;  // summary tiles loaded ahead of the one in use

template <int D, int RPW, int HT, int ECLS>
__device__ __forceinline__ void route_rows_body(const Geom& g, const RouteParams& p,
                                                uint8_t* __restrict__ flags, RrShared& sh) {
  constexpr int KS = D / 32;
  constexpr int R = kRrWaves * RPW;   // rows per workgroup
  constexpr int NH = 16 * HT;         // query heads per KV head
  static_assert(RPW * NH == 64, "one lane per (row, head) in the solve");
  auto& Cand = sh.cand;
  auto& Cnt = sh.cnt;
  auto& Bnd = sh.bnd;
  auto& Tau = sh.tau;

  const int tid = threadIdx.x, lane = tid & 63;
  const int wv = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int r = lane & 15, gq = lane >> 4;
  const int h = blockIdx.y;
  const int gps = (g.max_seqlen + R - 1) / R;  // row groups per sequence
  const int gi = blockIdx.x;
  const int s = gi / gps;
  const int pos0 = (gps - 1 - gi % gps) * R;   // costliest groups first
  const SeqInfo si = seq_info(g.cu_seqlens, g.cu_chunks, s, g.max_seqlen, g.B);
  if (pos0 >= si.len) return;
  const float alpha = p.alpha_per_seq ? p.alpha_per_seq[s] : p.alpha;
  const float am1 = alpha - 1.f;
  const float ex = 1.f / am1;
  const float xsc = p.gamma_scale * am1;  // logits straight to x units
  const int64_t rows = p.rows;

  // this wave's rows j < RPW: position, token row, routable chunks
  int pos[RPW], n[RPW];
  int64_t tok[RPW];
  int nmax = 0;
#pragma unroll
  for (int j = 0; j < RPW; ++j) {
    pos[j] = pos0 + wv * RPW + j;
    const bool valid = pos[j] < si.len;
    n[j] = valid ? pos[j] / g.B : 0;
    tok[j] = si.start + min(pos[j], si.len - 1);
    nmax = max(nmax, n[j]);
  }
  const int ntile = (nmax + 15) >> 4;
  // Q fragments: lane (gq, r) holds head 16 ht + r, dims 32 ks + 8 gq
  bf16x8 qa[RPW][HT][KS];
#pragma unroll
  for (int j = 0; j < RPW; ++j)
#pragma unroll
    for (int ht = 0; ht < HT; ++ht) {
      const uint16_t* qrow =
          (const uint16_t*)p.q + (tok[j] * g.Hq + h * g.G + 16 * ht + r) * (int64_t)D;
#pragma unroll
      for (int ks = 0; ks < KS; ++ks) qa[j][ht][ks] = as_bf16x8(ldg16(qrow + 32 * ks + 8 * gq));
    }
  // summary fragments of chunk tile t: lane (gq, r) holds chunk 16 t + r
  // (clamped to a routable chunk of the row group), dims 32 ks + 8 gq
  const uint16_t* kb = (const uint16_t*)p.kbar + ((si.chunk_off * g.Hkv + h) * (int64_t)D);
  const int64_t kstride = (int64_t)g.Hkv * D;
  const int clast = max(nmax - 1, 0);
  auto kload = [&](u32x4 (&f)[KS], int t) {
    const uint16_t* krow = kb + (int64_t)min(16 * t + r, clast) * kstride + 8 * gq;
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) f[ks] = ldg16(krow + 32 * ks);
  };
  // one pass over the chunk tiles: body(t, j, ht, a[4]) with a the logits of
  // heads 16 ht + 4 gq + jj, chunk 16 t + r, as accumulated (x = a * xsc)
  auto pass = [&](auto&& body) {
    if (ntile == 0) return;
    constexpr int NB = kRrAhead + 1;
    u32x4 kf[NB][KS];
#pragma unroll
    for (int a = 0; a < kRrAhead; ++a) {
      kload(kf[a], min(a, ntile - 1));
      // issued in tile order: the counted waits below assume it
      __builtin_amdgcn_sched_barrier(0);
    }
    // unrolled by the buffer count so that every buffer index is a constant;
    // the tiles are padded to a whole number of rounds (a tile past the end
    // holds no routable chunk of any row, so every body ignores it) so that
    // the loop body has no exit and the loads' counted waits stay exact
    for (int t0 = 0; t0 < ntile; t0 += NB) {
      static_for<0, NB>([&](auto u_) {
        constexpr int U = decltype(u_)::value;
        const int t = t0 + U;
        // the loads of tile t + kRrAhead (clamped: past the end the last
        // tile is loaded again)
        kload(kf[(U + kRrAhead) % NB], min(t + kRrAhead, ntile - 1));
        // (keeps the scheduler from sinking the loads next to their use,
        // which would undo the prefetch)
        __builtin_amdgcn_sched_barrier(0);
        // the RPW * HT accumulator chains interleaved (ks outermost), so no
        // MFMA waits on the one just issued
        f32x4 acc[RPW][HT];
#pragma unroll
        for (int j = 0; j < RPW; ++j)
#pragma unroll
          for (int ht = 0; ht < HT; ++ht) acc[j][ht] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int ks = 0; ks < KS; ++ks)
#pragma unroll
          for (int j = 0; j < RPW; ++j)
#pragma unroll
            for (int ht = 0; ht < HT; ++ht)
              acc[j][ht] = mfma16x16x32(qa[j][ht][ks], as_bf16x8(kf[U][ks]), acc[j][ht]);
#pragma unroll
        for (int j = 0; j < RPW; ++j)
#pragma unroll
          for (int ht = 0; ht < HT; ++ht) {
            float a[4];
#pragma unroll
            for (int jj = 0; jj < 4; ++jj) a[jj] = acc[j][ht][jj];
            body(t, j, ht, a);
          }
      });
    }
  };

  // ---- 1. partial maxima, then the lower bound b per (row, head)
  float mx[RPW][HT][4];
#pragma unroll
  for (int j = 0; j < RPW; ++j)
#pragma unroll
    for (int ht = 0; ht < HT; ++ht)
#pragma unroll
      for (int jj = 0; jj < 4; ++jj) mx[j][ht][jj] = -INFINITY;
  // (the maximum of the accumulated logits, scaled once after the pass: the
  // scale is positive, so this is the maximum of the scaled ones)
  pass([&](int t, int j, int ht, const float (&a)[4]) {
    const bool ok = 16 * t + r < n[j];
#pragma unroll
    for (int jj = 0; jj < 4; ++jj) mx[j][ht][jj] = fmaxf(mx[j][ht][jj], ok ? a[jj] : -INFINITY);
  });
  // the 16 lanes of a lane group hold one (row, head)'s partial maxima
#pragma unroll
  for (int j = 0; j < RPW; ++j)
#pragma unroll
    for (int ht = 0; ht < HT; ++ht)
#pragma unroll
      for (int jj = 0; jj < 4; ++jj) {
        const float v = mx[j][ht][jj] * xsc;
        const float top = row16_max(v);
        float b = top - 1.f;  // the top value alone has mass 1 here
#pragma unroll
        for (int it = 0; it < kRrBoundIters; ++it) {
          float pw, pd;
          rr_pow<ECLS>(fmaxf(v - b, 0.f), ex, pw, pd);
          const float f = row16_sum(pw), fd = row16_sum(pd);
          const float step = (f - 1.f) / (ex * fd);
          b = (step > 0.f && fd > 0.f) ? b + step : b;
        }
        // Newton from below stays below the 16-value root up to rounding;
        // the margin keeps b below it (a few more candidates at most)
        b -= 1e-4f * fmaxf(1.f, fabsf(b));
        b = n[j] > 0 ? b : INFINITY;
        mx[j][ht][jj] = b;
      }

  // ---- 2. candidate lists: every x > b of the (row, head)
  int cnt[RPW][HT][4];
#pragma unroll
  for (int j = 0; j < RPW; ++j)
#pragma unroll
    for (int ht = 0; ht < HT; ++ht)
#pragma unroll
      for (int jj = 0; jj < 4; ++jj) cnt[j][ht][jj] = 0;
  const uint32_t below = (1u << r) - 1u;
  // the bound in accumulated units: x > tau implies x > b plus the bound's
  // margin, far above the rounding of either scaling, so comparing a with
  // b / xsc still keeps every x > tau
  float braw[RPW][HT][4];
#pragma unroll
  for (int j = 0; j < RPW; ++j)
#pragma unroll
    for (int ht = 0; ht < HT; ++ht)
#pragma unroll
      for (int jj = 0; jj < 4; ++jj) braw[j][ht][jj] = mx[j][ht][jj] / xsc;
  pass([&](int t, int j, int ht, const float (&a)[4]) {
    const bool ok = 16 * t + r < n[j];
    // (the ballots of the bare compares, masked by the chunk range on the
    // scalar side: a ballot of the combined condition costs two more vector
    // instructions an element)
    const uint64_t okm = __builtin_amdgcn_ballot_w64(ok);
#pragma unroll
    for (int jj = 0; jj < 4; ++jj) {
      const bool gt = a[jj] > braw[j][ht][jj];
      const bool c = ok && gt;
      const uint32_t grp =
          (uint32_t)((__builtin_amdgcn_ballot_w64(gt) & okm) >> (16 * gq)) & 0xffffu;
      // past the capacity: the row's pad word (the count records the overflow)
      const int slot = ::min(cnt[j][ht][jj] + (int)__popc(grp & below), kRrCap);
      if (c) Cand[wv][j * NH + 16 * ht + 4 * gq + jj][slot] = a[jj] * xsc;
      cnt[j][ht][jj] += __popc(grp);
    }
  });
  // rows with an overflowing list are left to the fallback (flag 1)
  bool ovr[RPW];
#pragma unroll
  for (int j = 0; j < RPW; ++j) {
    bool over = false;
#pragma unroll
    for (int ht = 0; ht < HT; ++ht)
#pragma unroll
      for (int jj = 0; jj < 4; ++jj) {
        over = over || cnt[j][ht][jj] > kRrCap;
        if (r == 0) {
          Cnt[wv][j * NH + 16 * ht + 4 * gq + jj] = min(cnt[j][ht][jj], kRrCap);
          Bnd[wv][j * NH + 16 * ht + 4 * gq + jj] = mx[j][ht][jj];
        }
      }
    ovr[j] = __ballot(over) != 0ull;
    if (lane == 0 && pos[j] < si.len) flags[(int64_t)h * route_flag_stride(rows) + tok[j]] = ovr[j] ? 1 : 0;
  }

  // ---- 3a. thresholds: lane l solves (row l / NH, head l % NH) on its list,
  // held in registers (groups of 8 up to the wave's longest list; entries past
  // the lane's own list are -inf and add nothing)
  {
    const int m = Cnt[wv][lane];
    const float* cl = Cand[wv][lane];
    int mmax = m;  // the wave's longest list
#pragma unroll
    for (int o = 32; o > 0; o >>= 1) mmax = max(mmax, __shfl_xor(mmax, o));
    mmax = __builtin_amdgcn_readfirstlane(mmax);
    constexpr int NG8 = kRrCap / 8;
    float xv[kRrCap];
#pragma unroll
    for (int i = 0; i < kRrCap; ++i) xv[i] = (i < mmax && i < m) ? cl[i] : -INFINITY;
    const int ng = (mmax + 7) >> 3;
    float tau = Bnd[wv][lane];
    bool rovr = false;
#pragma unroll
    for (int j = 0; j < RPW; ++j) rovr = rovr || (lane / NH == j && ovr[j]);
    const bool live = tau != INFINITY && !rovr;
    bool done = !live;
    for (int it = 0; it < 100; ++it) {
      if (__ballot(!done) == 0ull) break;
      float f = 0.f, fd = 0.f;
#pragma unroll
      for (int g8 = 0; g8 < NG8; ++g8) {
        if (g8 < ng) {
#pragma unroll
          for (int i = 8 * g8; i < 8 * g8 + 8; ++i) {
            float pw, pd;
            rr_pow<ECLS>(fmaxf(xv[i] - tau, 0.f), ex, pw, pd);
            f += pw;
            fd += pd;
          }
        }
      }
      if (!done) {
        const float step = (f - 1.f) / (ex * fd);
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
      // 1.5-entmax tau = M - sqrt((1 - sum_S (x - M)^2) / |S|), M the mean over S
      float s1 = 0.f, c1 = 0.f, mn_in = INFINITY, mx_out = -INFINITY;
#pragma unroll
      for (int g8 = 0; g8 < NG8; ++g8) {
        if (g8 < ng) {
#pragma unroll
          for (int i = 8 * g8; i < 8 * g8 + 8; ++i) {
            const bool in = xv[i] > tau;
            s1 += in ? xv[i] : 0.f;
            c1 += in ? 1.f : 0.f;
            mn_in = fminf(mn_in, in ? xv[i] : INFINITY);
            mx_out = fmaxf(mx_out, in ? -INFINITY : xv[i]);
          }
        }
      }
      // values left off the list lie at or below b <= tau
      mx_out = fmaxf(mx_out, live ? Bnd[wv][lane] : -INFINITY);
      float t2;
      if constexpr (ECLS == 1) {
        t2 = (s1 - 1.f) / c1;
      } else {
        const float M = s1 / c1;
        float q2 = 0.f;
#pragma unroll
        for (int g8 = 0; g8 < NG8; ++g8) {
          if (g8 < ng) {
#pragma unroll
            for (int i = 8 * g8; i < 8 * g8 + 8; ++i) {
              const float dm = xv[i] > tau ? xv[i] - M : 0.f;
              q2 = fmaf(dm, dm, q2);
            }
          }
        }
        t2 = M - sqrtf(fmaxf(0.f, (1.f - q2) / c1));
      }
      if (live && c1 > 0.f && t2 < mn_in && t2 >= mx_out) tau = t2;
    }
    Tau[wv][lane] = tau;
    const int pj = pos0 + wv * RPW + lane / NH;
    if (p.tau && pj < si.len && !rovr)
      p.tau[(int64_t)(h * g.G + lane % NH) * rows + si.start + pj] = live ? tau / am1 : INFINITY;
  }
  // (the wave reads back its own lanes' thresholds: LDS ops of a wave are in order)

  // ---- 3b. weights, mask words and log-prior, one chunk tile at a time
  float tq[RPW][HT][4];
#pragma unroll
  for (int j = 0; j < RPW; ++j)
#pragma unroll
    for (int ht = 0; ht < HT; ++ht)
#pragma unroll
      for (int jj = 0; jj < 4; ++jj) tq[j][ht][jj] = Tau[wv][j * NH + 16 * ht + 4 * gq + jj];
  const float invG = 1.f / (float)g.G;
  uint64_t word[RPW];
  float wsum[RPW];
#pragma unroll
  for (int j = 0; j < RPW; ++j) word[j] = 0ull;
  // After the reduce-scatter below, lane group gq holds the sums of row rr:
  // rows 0, 2, 1, 3 for lane groups 0 .. 3 (four rows a wave), rows 0, 1, 0, 1
  // (two rows a wave: lane groups 0 and 1 store them)
  const int rr = RPW == 4 ? 2 * (gq & 1) + (gq >> 1) : (gq & 1);
  int nr = n[0];
  int64_t tr = tok[0];
  bool ovr_r = ovr[0];
#pragma unroll
  for (int j = 1; j < RPW; ++j) {
    nr = rr == j ? n[j] : nr;
    tr = rr == j ? tok[j] : tr;
    ovr_r = rr == j ? ovr[j] : ovr_r;
  }
  const bool writer = RPW == 4 || (gq & 2) == 0;
  pass([&](int t, int j, int ht, const float (&a)[4]) {
    if (ht == 0) wsum[j] = 0.f;
#pragma unroll
    for (int jj = 0; jj < 4; ++jj) {
      const float d = a[jj] * xsc - tq[j][ht][jj];
      float pw, pd;
      rr_pow<ECLS>(fmaxf(d, 0.f), ex, pw, pd);
      wsum[j] += pw;
    }
    if (j != RPW - 1 || ht != HT - 1) return;
    // every row's sum over the four lane groups (the group's heads), as a
    // reduce-scatter: each lane group keeps half of its rows and adds the
    // partner group's half (lane l ^ 16), then the same across l ^ 32.  The
    // additions are those of a per-row sum in the fixed order (g0 + g1) +
    // (g2 + g3) up to commutativity, so every row gets the same bits as from
    // an all-reduce, with one ballot, one log and one store for all rows.
    float w;
    const bool od = (gq & 1) != 0;
    if constexpr (RPW == 4) {
      const float k0 = od ? wsum[2] : wsum[0], k1 = od ? wsum[3] : wsum[1];
      const float s0 = od ? wsum[0] : wsum[2], s1 = od ? wsum[1] : wsum[3];
      const float a0 = k0 + xor16(s0), a1 = k1 + xor16(s1);
      const bool hi = (gq & 2) != 0;
      w = (hi ? a1 : a0) + xor32(hi ? a0 : a1);
    } else {
      const float a0 = (od ? wsum[1] : wsum[0]) + xor16(od ? wsum[0] : wsum[1]);
      w = a0 + xor32(a0);
    }
    // the chunk is active iff some head's weight is positive
    const int c = 16 * t + r;
    const bool on = w > 0.f && c < nr;
    const uint64_t bits = __builtin_amdgcn_ballot_w64(on);
    if (p.log_prior && writer && c < nr && !ovr_r)
      p.log_prior[((int64_t)h * rows + tr) * g.C_slots + c] =
          on ? (p.sigma == 0.f ? 0.f : p.sigma * logf(fmaxf(w * invG, 1e-38f))) : -INFINITY;
#pragma unroll
    for (int jr = 0; jr < RPW; ++jr) {
      // row jr's 16 chunks are the bits of the lane group holding it
      const int gj = RPW == 4 ? ((jr & 1) << 1) | (jr >> 1) : jr;
      word[jr] |= ((bits >> (16 * gj)) & 0xffffull) << (16 * (t & 3));
    }
    if (((t & 3) == 3 || t == ntile - 1) && t < ntile) {
#pragma unroll
      for (int jr = 0; jr < RPW; ++jr) {
        if (lane == 0 && pos[jr] < si.len && !ovr[jr])
          p.mask[((int64_t)h * rows + tok[jr]) * g.W + (t >> 2)] = word[jr];
        word[jr] = 0ull;
      }
    }
  });
  // words past the last tile's
#pragma unroll
  for (int j = 0; j < RPW; ++j) {
    if (pos[j] >= si.len || ovr[j]) continue;
    for (int w = ((ntile + 3) >> 2) + lane; w < g.W; w += 64)
      p.mask[((int64_t)h * rows + tok[j]) * g.W + w] = 0ull;
  }
}

// ECLS < 0: the exponent 1/(alpha - 1) is the sequence's (alpha per
// sequence), its form chosen here per workgroup.
template <int D, int RPW, int HT, int ECLS>
__global__ __launch_bounds__(64 * kRrWaves) void route_rows_kernel(Geom g, RouteParams p,
                                                                 uint8_t* __restrict__ flags) {
  __shared__ RrShared sh;
  if constexpr (ECLS >= 0) {
    route_rows_body<D, RPW, HT, ECLS>(g, p, flags, sh);
  } else {
    const int R = kRrWaves * RPW;
    const int gps = (g.max_seqlen + R - 1) / R;
    const float a = p.alpha_per_seq[blockIdx.x / gps];
    const float e = 1.f / (a - 1.f);
    if (!(a > 1.f)) {  // softmax routing: the fallback routes the group's rows
      const int s = blockIdx.x / gps;
      const int pos0 = (gps - 1 - blockIdx.x % gps) * R;
      const SeqInfo si = seq_info(g.cu_seqlens, g.cu_chunks, s, g.max_seqlen, g.B);
      const int i = pos0 + threadIdx.x;
      if (threadIdx.x < R && i < si.len) flags[(int64_t)blockIdx.y * route_flag_stride(p.rows) + si.start + i] = 1;
      return;
    }
    if (e == 1.f) route_rows_body<D, RPW, HT, 1>(g, p, flags, sh);
    else if (e == 2.f) route_rows_body<D, RPW, HT, 2>(g, p, flags, sh);
    else if (e == 4.f) route_rows_body<D, RPW, HT, 4>(g, p, flags, sh);
    else route_rows_body<D, RPW, HT, 0>(g, p, flags, sh);
  }
}

bool route_rows_supported(const Geom& g, const RouteParams& p) {
  return g.bf16 && !p.seqlens && !p.kdiag && p.topk <= 0 && (g.G == 16 || g.G == 32) &&
         (p.alpha > 1.f || p.alpha_per_seq) && p.row0 == 0 && p.rows == g.T;
}

int route_rows_per_group(const Geom& g) { return kRrWaves * (g.G == 32 ? 2 : 4); }

int64_t route_rows_flag_bytes(const Geom& g) { return route_flag_stride(g.T) * g.Hkv; }

hipError_t launch_route_rows(const Geom& g, const RouteParams& p, uint8_t* flags,
                             hipStream_t st) {
  const int RPW = g.G == 32 ? 2 : 4;
  const int R = kRrWaves * RPW;
  const int gps = (g.max_seqlen + R - 1) / R;
  dim3 grid((unsigned)(g.num_seqs * gps), g.Hkv);
  // alpha_per_seq: the exponent's form is chosen per workgroup (-1)
  const float ex = 1.f / (p.alpha - 1.f);
  const int ecls = p.alpha_per_seq ? -1 : (ex == 1.f ? 1 : (ex == 2.f ? 2 : (ex == 4.f ? 4 : 0)));
#define DASH_RR(DD, RP, H, E) \
  hipLaunchKernelGGL((route_rows_kernel<DD, RP, H, E>), grid, dim3(64 * kRrWaves), 0, st, g, p, flags)
#define DASH_RR_E(DD, RP, H)                   \
  do {                                         \
    if (ecls == 1) DASH_RR(DD, RP, H, 1);      \
    else if (ecls == 2) DASH_RR(DD, RP, H, 2); \
    else if (ecls == 4) DASH_RR(DD, RP, H, 4); \
    else if (ecls == 0) DASH_RR(DD, RP, H, 0); \
    else DASH_RR(DD, RP, H, -1);               \
  } while (0)
  if (g.D == 64) {
    if (g.G == 32) DASH_RR_E(64, 2, 2); else DASH_RR_E(64, 4, 1);
  } else {
    if (g.G == 32) DASH_RR_E(128, 2, 2); else DASH_RR_E(128, 4, 1);
  }
#undef DASH_RR_E
#undef DASH_RR
  return hipGetLastError();
}

}  // namespace dash
