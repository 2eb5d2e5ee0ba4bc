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
// kbar_t_kernel: K_bar transposed per sequence and KV head, [D][C padded to
// 32] bf16, the B operand of du K_bar.
// route_bwd_kernel (one workgroup per row and KV head): recomputes the row's
// logits (MFMA) and, from the forward's thresholds, each head's p; forms
// w_bar, dp, and per head r, rho and du (in LDS); adds gamma s du K_bar to dq
// (MFMA, du rounded to bf16); stores dp (over db) and each head's
// (threshold, softmax sum, rho) for the chunk pass.
// kbar_grad_kernel (one workgroup per 64 chunks, KV head and slice of rows):
// walks the rows that route to any of its chunks, recomputes their logits
// and du for its chunks (the same MFMA, so the same r as above), and
// accumulates dk_bar = gamma s du^T Q (MFMA); slices meet by atomics.
// kbar_sum_bwd_kernel (one workgroup per complete chunk and KV head): the
// summary's backward into dk and dq_bar.
// With estimate_diagonal, route_bwd_kernel also differentiates each row's
// own-chunk entry (du_d = -r_d rho: it feeds no prior) into dq and the
// estimate's gradient, and diag_sum_bwd_kernel takes that back through the
// running summaries into dk and dq_bar.
// bf16, G = 16 or 32; fixed-length or packed (varlen) sequences.
#include "dash_device.h"
#include "dash_internal.h"

#include <algorithm>

namespace dash {

// d^e for d >= 0 (0 at d = 0 unless e = 0, where it is the support indicator);
// the exponents of alpha = 1.5 (1 and 2) and alpha = 2 (0 and 1) directly
__device__ __forceinline__ float pow_pos(float d, float e) {
  if (!(d > 0.f)) return 0.f;
  if (e == 1.f) return d;
  if (e == 2.f) return d * d;
  if (e == 0.f) return 1.f;
  return exp2f(e * __log2f(d));
}

// K_bar^T: kbt[((s Hkv + h) D + d) cpad + c], zero past the sequence's chunks
__global__ __launch_bounds__(256) void kbar_t_kernel(Geom g, const uint16_t* __restrict__ kbar,
                                                     uint16_t* __restrict__ kbt, int cpad) {
  const int64_t idx = (int64_t)blockIdx.x * 256 + threadIdx.x;
  const int64_t n = (int64_t)g.num_seqs * g.Hkv * g.D * cpad;
  if (idx >= n) return;
  const int c = (int)(idx % cpad);
  const int64_t r = idx / cpad;
  const int d = (int)(r % g.D);
  const int sh = (int)(r / g.D);
  const int h = sh % g.Hkv, s = sh / g.Hkv;
  const SeqInfo si = seq_info(g.cu_seqlens, g.cu_chunks, s, g.max_seqlen, g.B);
  uint16_t v = 0;
  if (c < si.len / g.B) v = kbar[((si.chunk_off + c) * g.Hkv + h) * g.D + d];
  kbt[idx] = v;
}

// wide = 0: the rows whose entries fit CP (every row's flag written: 1 for a
// row left to the wide pass); wide = 1: only the rows flagged so.
template <int D, int CP>
__global__ __launch_bounds__(256, CP == 256 ? 7 : 1) void route_bwd_kernel(Geom g, RouteBwdParams p, int row0,
                                                        int row1, int wide) {
  constexpr int NTH = 256;
  constexpr int KS = D / 32;
  constexpr int USTR = CP + 16;
  __shared__ __align__(16) float U[16 * USTR];   // logits, then du, of one 16-head tile
  __shared__ float Wp[CP];         // sum over the group's heads of p, then dp
  __shared__ uint8_t On[CP];       // the entry's chunk is active
  __shared__ uint16_t L[CP];       // the row's entries: chunk of entry k
  __shared__ int Wpre[33];         // entries before each mask word
  __shared__ float Hp[16][2];      // per head: threshold (x units) or max u; softmax sum
  __shared__ float Dd[16];         // per head: du of the own-chunk entry
  const int row = row0 + (int)blockIdx.x, h = blockIdx.y;
  if (row >= row1) return;
  const int tid = threadIdx.x, lane = tid & 63, wv = tid >> 6;
  const int r = lane & 15, gq = lane >> 4;
  const int64_t T = g.T;
  const int s = g.cu_seqlens ? find_seq(g.cu_seqlens, g.num_seqs, row) : row / g.max_seqlen;
  const SeqInfo si = seq_info(g.cu_seqlens, g.cu_chunks, s, g.max_seqlen, g.B);
  const int pos = (int)(row - si.start);
  const int64_t kb0 = si.chunk_off;
  const int n = pos / g.B;
  const int G = g.G;
  float4* sc = p.sc;
  uint8_t* rflag = p.rflags + (int64_t)h * route_flag_stride(T) + row;
  if (wide && *rflag == 0) return;
  if (n == 0) {
    if (tid == 0) *rflag = 0;
    if (tid < G) sc[(int64_t)(h * G + tid) * T + row] = make_float4(0.f, 0.f, 0.f, 0.f);
    if (p.kdiag && tid < D) p.dkdiag[((int64_t)row * g.Hkv + h) * D + tid] = 0.f;
    return;
  }
  const float alpha = p.alpha_per_seq ? p.alpha_per_seq[s] : p.alpha;
  const bool smax = !(alpha > 1.f);
  const float am1 = alpha - 1.f;
  const float ep = smax ? 1.f : 1.f / am1;            // p = d^ep
  const float er = smax ? 1.f : (2.f - alpha) / am1;  // r = d^er
  const int HT = G / 16;

  // ---- the row's entries.  alpha > 1: only the chunks the mask holds (every
  // head's support lies in the union the mask is, so p, r and du vanish on
  // the others); softmax: every routable chunk (every p > 0).  With
  // estimate_diagonal the own-chunk estimate is one more entry, last.
  const unsigned long long* mrow = p.mask + ((int64_t)h * T + row) * g.W;
  const int nw = (n + 63) >> 6;
  if (tid < 64) {
    const unsigned long long wd = tid < nw ? mrow[tid] & routable_bits(tid, n) : 0ull;
    const int cnt = smax ? max(0, min(64, n - 64 * tid)) : __popcll(wd);
    int inc = cnt;
#pragma unroll
    for (int o = 1; o < 64; o <<= 1) {
      const int y = __shfl_up(inc, o);
      if (lane >= o) inc += y;
    }
    if (tid < 33) Wpre[tid] = inc - cnt;
    if (tid < nw) {
      int o = inc - cnt;
      if (smax) {
        for (int b = 0; b < cnt && o + b < CP; ++b) {
          L[o + b] = (uint16_t)(64 * tid + b);
          On[o + b] = (uint8_t)((wd >> b) & 1ull);
        }
      } else {
        unsigned long long v = wd;
        while (v && o < CP) {  // (a longer list leaves the row to the wide pass)
          L[o] = (uint16_t)(64 * tid + __ffsll((long long)v) - 1);
          On[o++] = 1;
          v &= v - 1;
        }
      }
    }
  }
  __syncthreads();
  const int na = Wpre[nw];                  // listed chunks
  if (!wide) {
    // more entries than this pass holds: left to the wide pass
    if (tid == 0) *rflag = na > CP ? 1 : 0;
    if (na > CP) return;
  }
  const int ns = p.kdiag ? na + 1 : na;     // entries
  const int n32 = (na + 31) & ~31;
  const uint16_t* kdrow = (const uint16_t*)p.kdiag + ((int64_t)row * g.Hkv + h) * D;

  // logits of head tile ht for the entries into U (16 heads x ns, MFMA)
  auto logits = [&](int ht) {
    const uint16_t* qrow = (const uint16_t*)p.q + (((int64_t)row * g.Hq + h * G + 16 * ht + r) * D);
    bf16x8 qa[KS];
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) qa[ks] = as_bf16x8(ldg16(qrow + 32 * ks + 8 * gq));
    const int nct = (ns + 15) >> 4;
    for (int ct = wv; ct < nct; ct += 4) {
      const int k = min(ct * 16 + r, ns - 1);
      const uint16_t* krow =
          k == na ? kdrow : (const uint16_t*)p.kbar + (((kb0 + L[k]) * g.Hkv + h) * (int64_t)D);
      f32x4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int ks = 0; ks < KS; ++ks)
        acc = mfma16x16x32(qa[ks], as_bf16x8(ldg16(krow + 32 * ks + 8 * gq)), acc);
      if (ct * 16 + r < ns) {
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
      for (int c = r; c < ns; c += 16) mx = fmaxf(mx, ur[c]);
      mx = row16_max(mx);
      float z = 0.f;
      for (int c = r; c < ns; c += 16) z += exp2f((ur[c] - mx) * kLog2e);
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
  for (int k = tid; k < na; k += NTH) Wp[k] = 0.f;
  for (int ht = 0; ht < HT; ++ht) {
    __syncthreads();
    logits(ht);
    __syncthreads();
    head_params(ht);
    __syncthreads();
    for (int k = tid; k < na; k += NTH) {
      float w = 0.f;
#pragma unroll 4
      for (int hh = 0; hh < 16; ++hh) w += prob(U[hh * USTR + k], hh);
      Wp[k] += w;
    }
  }
  __syncthreads();
  // ---- dp on the active chunks (written over db).  A chunk the mask holds
  // but whose recomputed w_bar is 0 (every head's logit within rounding of
  // its threshold: the mask's kernel forms the logits in another order) has
  // r = 0 for every head below, so it carries no gradient: dp = 0 there.
  float* drow = p.db + ((int64_t)h * T + row) * g.C_slots;
  for (int k = tid; k < na; k += NTH) {
    const int c = L[k];
    const float dp = (On[k] && Wp[k] > 0.f) ? p.sigma * drow[c] / Wp[k] : 0.f;
    Wp[k] = dp;
    drow[c] = dp;
  }
  // ---- pass 2 per head tile: r, rho, du; dq += gamma s du K_bar
  float dkd = 0.f;  // thread tid < D: dim tid of the estimate's gradient
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
      for (int k = r; k < na; k += 16) {
        const float rr = On[k] ? rterm(ur[k], hh) : 0.f;
        num = fmaf(rr, Wp[k], num);
        den += rr;
      }
      // the own-chunk entry: in the entmax, no prior (its dp is 0)
      const float rd = (p.kdiag && r == 0) ? rterm(ur[na], hh) : 0.f;
      den += rd;
      num = row16_sum(num);
      den = row16_sum(den);
      const float rho = den > 0.f ? num / den : 0.f;
      if (p.kdiag && r == 0) Dd[hh] = -rd * rho;
      // every lane of the head has read its U entries above; du overwrites them
      for (int k = r; k < n32; k += 16) {
        float du = 0.f;
        if (k < na && On[k]) du = rterm(ur[k], hh) * (Wp[k] - rho);
        ur[k] = du;
      }
      if (r == 0)
        sc[(int64_t)(h * G + 16 * ht + hh) * T + row] = make_float4(Hp[hh][0], Hp[hh][1], rho, 0.f);
    }
    __syncthreads();
    // dq tile (16 heads x 16 dims) = du (16 x n32) K_bar (n32 x 16) over the
    // listed chunks, the B operand gathered from K_bar^T; wave wv: dim tiles
    // wv, wv + 4
    constexpr int NT = D / 16;
    const uint16_t* kt = p.kbt + ((int64_t)(s * g.Hkv + h) * D) * p.cpad;
    for (int dt = wv; dt < NT; dt += 4) {
      f32x4 acc = {0.f, 0.f, 0.f, 0.f};
      const uint16_t* ktr = kt + (int64_t)(16 * dt + r) * p.cpad;
      const float* ua = U + r * USTR + 8 * gq;
      for (int c0 = 0; c0 < n32; c0 += 32) {
        const f32x4 a0 = *reinterpret_cast<const f32x4*>(ua + c0);
        const f32x4 a1 = *reinterpret_cast<const f32x4*>(ua + c0 + 4);
        const u32x4 av = {cvt_pk_bf16(a0[0], a0[1]), cvt_pk_bf16(a0[2], a0[3]),
                          cvt_pk_bf16(a1[0], a1[1]), cvt_pk_bf16(a1[2], a1[3])};
        // entries past the list carry du = 0: any listed chunk serves there
        u32x4 bv;
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const int k0 = min(c0 + 8 * gq + 2 * i, na - 1);
          const int k1 = min(c0 + 8 * gq + 2 * i + 1, na - 1);
          bv[i] = (uint32_t)ktr[L[k0]] | ((uint32_t)ktr[L[k1]] << 16);
        }
        acc = mfma16x16x32(as_bf16x8(av), as_bf16x8(bv), acc);
      }
      // lane (gq, r): heads 16 ht + 4 gq + j, dim 16 dt + r
      const float kd = p.kdiag ? bf16_to_f32(kdrow[16 * dt + r]) : 0.f;
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        float* dq = p.dq + ((int64_t)row * g.Hq + h * G + 16 * ht + 4 * gq + j) * D + 16 * dt + r;
        const float add = p.kdiag ? fmaf(Dd[4 * gq + j], kd, acc[j]) : acc[j];
        *dq += p.gamma_scale * add;
      }
    }
    // the estimate's gradient: gamma s sum over the tile's heads of du_d q
    if (p.kdiag && tid < D) {
      const uint16_t* qh = (const uint16_t*)p.q + ((int64_t)row * g.Hq + h * G + 16 * ht) * D + tid;
#pragma unroll 4
      for (int hh = 0; hh < 16; ++hh) dkd = fmaf(Dd[hh], bf16_to_f32(qh[hh * D]), dkd);
    }
  }
  if (p.kdiag && tid < D) p.dkdiag[((int64_t)row * g.Hkv + h) * D + tid] = p.gamma_scale * dkd;
}

// dk_bar of 64 chunks: rows that route to any of them, in slices over
// blockIdx.y.  Wave w owns chunks c0 + 16 w .. +15 (their K_bar rows as the B
// operand of the logits).  The slice's rows with any of the 64 chunks active
// are compacted from the mask words, and each such row's Q (all G heads, in
// 16-byte pieces swizzled by head_row_swz), its heads' stored (threshold,
// softmax sum, rho) and its dp of the 64 chunks stream through a ring of LDS
// stages by direct global->LDS loads, several rows ahead of the one computed
// (no plain load in the loop: the compiler would wait for the whole ring).
// Per row and head tile: u = Q K_bar^T (16x16x32), du from the stored terms,
// dk_bar^T += du^T Q (16x16x16, Q's transpose by transposing LDS reads).
template <int D, int HT>
__global__ __launch_bounds__(256) void kbar_grad_kernel(Geom g, RouteBwdParams p) {
  constexpr int NTH = 256;
  constexpr int G = 16 * HT;
  constexpr int KS = D / 32;
  constexpr int NT = D / 16;
  constexpr int UPH = D / 8;               // 16-byte pieces per head row
  constexpr int ABYTES = G * D * 2;        // one row's Q
  constexpr int PPW = ABYTES / 16 / 4;     // pieces per wave per row
  constexpr int NOP = (PPW + 63) / 64;     // 16-byte loads per wave per row
  constexpr int PER = NOP + 2;             // + the heads' terms and the chunks' dp
  constexpr int NSR = 4;                   // ring stages, one row each
  __shared__ __align__(16) uint8_t Ring[NSR][ABYTES];
  __shared__ __align__(16) float4 Sc[NSR][G];
  __shared__ __align__(16) float Dp[NSR][64];
  __shared__ int Rows[NTH];
  __shared__ unsigned long long Words[NTH];
  __shared__ int Wcnt[NTH / 64];
  const int tile = blockIdx.x;
  const int h = blockIdx.z % g.Hkv, s = blockIdx.z / g.Hkv;
  const int tid = threadIdx.x, lane = tid & 63;
  const int wv = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int r = lane & 15, gq = lane >> 4;
  const SeqInfo si = seq_info(g.cu_seqlens, g.cu_chunks, s, g.max_seqlen, g.B);
  const int len = si.len;
  const int cs = len / g.B;
  const int c0 = tile * 64;
  if (c0 >= cs) return;
  const int64_t T = g.T;
  const int64_t start = si.start;
  const int64_t kb0 = si.chunk_off;
  // rows that may route to the tile: n(i) > c0
  const int rbeg = (c0 + 1) * g.B;
  const int per = (len - rbeg + (int)gridDim.y - 1) / (int)gridDim.y;
  const int rlo = rbeg + (int)blockIdx.y * per;
  const int rhi = min(len, rlo + per);
  if (rlo >= rhi) return;
  const float alpha = p.alpha_per_seq ? p.alpha_per_seq[s] : p.alpha;
  const float am1 = alpha - 1.f;
  const bool smax = !(alpha > 1.f);
  const float er = smax ? 1.f : (2.f - alpha) / am1;
  const float gs = p.gamma_scale;

  // this wave's 16 chunks as the B operand of Q K_bar^T
  const int myc = c0 + 16 * wv + r;
  bf16x8 kb[KS];
  {
    const uint16_t* krow =
        (const uint16_t*)p.kbar + ((kb0 + min(myc, cs - 1)) * g.Hkv + h) * (int64_t)D;
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) kb[ks] = as_bf16x8(ldg16(krow + 32 * ks + 8 * gq));
  }
  // the operand loads complete here, so that the compiler's own waits for
  // them do not land in the ring loop
  wait_vm<0>();
  f32x4 acc[NT];
#pragma unroll
  for (int nt = 0; nt < NT; ++nt) acc[nt] = f32x4{0.f, 0.f, 0.f, 0.f};

  // one row into ring slot `slot`: every wave issues PER loads
  const int cpw = min(c0 + 16 * wv + lane, g.C_slots - 1);  // lane < 16: its dp word
  auto issue = [&](int row, int slot) {
    const int64_t tok = start + row;
    const uint32_t base = lds_addr(&Ring[slot][0]);
#pragma unroll
    for (int e = 0; e < NOP; ++e) {
      const int pl = 64 * e + lane;  // piece of this wave
      if (pl < PPW) {
        const int u = wv * PPW + pl;
        const int j = u / UPH, pc = (u % UPH) ^ head_row_swz<D>(j);
        lds_dma16((const uint16_t*)p.q + (tok * g.Hq + h * G + j) * (int64_t)D + 8 * pc,
                  __builtin_amdgcn_readfirstlane(base + (uint32_t)(16 * (wv * PPW + 64 * e))));
      }
    }
    if (lane < G / 4)
      lds_dma16(p.sc + (int64_t)(h * G + (G / 4) * wv + lane) * T + tok,
                __builtin_amdgcn_readfirstlane(lds_addr(&Sc[slot][(G / 4) * wv])));
    if (lane < 16)
      lds_dma4(p.db + ((int64_t)h * T + tok) * g.C_slots + cpw,
               __builtin_amdgcn_readfirstlane(lds_addr(&Dp[slot][16 * wv])));
  };
  // transposing reads: lane (gq, r) points at head 16 ht + 4 gq + r / 4,
  // dims 16 nt + 4 (r % 4) .. +3 and receives dim 16 nt + r of heads
  // 16 ht + 4 gq .. +3
  auto compute = [&](int slot, unsigned long long wbits) {
    lds_u8* qs = (lds_u8*)&Ring[slot][0];
    // dp of this lane's chunk (0 where the chunk is not active)
    const bool act = (wbits >> (16 * wv + r)) & 1ull;
    const float dp = act ? Dp[slot][16 * wv + r] : 0.f;
#pragma unroll
    for (int ht = 0; ht < HT; ++ht) {
      const int j = 16 * ht + r;
      f32x4 u = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int ks = 0; ks < KS; ++ks) {
        const u32x4 qa = lds_read16(qs + 16 * (j * UPH + ((4 * ks + gq) ^ head_row_swz<D>(j))));
        u = mfma16x16x32(as_bf16x8(qa), kb[ks], u);
      }
      // lane (gq, r): heads 16 ht + 4 gq + jj, chunk myc
      float du[4];
#pragma unroll
      for (int jj = 0; jj < 4; ++jj) {
        const float4 t = Sc[slot][16 * ht + 4 * gq + jj];
        const float x = u[jj] * gs;
        const float rr = smax ? exp2f((x - t.x) * kLog2e) / t.y : pow_pos(x * am1 - t.x, er);
        du[jj] = act ? rr * (dp - t.z) : 0.f;
      }
      const u32x2 da = {cvt_pk_bf16(du[0], du[1]), cvt_pk_bf16(du[2], du[3])};
      const int jt = 16 * ht + 4 * gq + (r >> 2);
      const int tb = 16 * jt * UPH + 16 * ((r & 3) >> 1) + 8 * (r & 1);
      const int tx = head_row_swz<D>(jt);
#pragma unroll
      for (int nt = 0; nt < NT; ++nt) {
        const s16x4 qb = lds_read_tr8(qs + tb + 16 * ((2 * nt) ^ tx));
        acc[nt] = mfma16x16x16(as_s16x4(da), qb, acc[nt]);
      }
    }
  };

  for (int r0 = rlo; r0 < rhi; r0 += NTH) {
    // rows r0 .. r0+255 with any of the tile's chunks active, compacted in order
    const int i = r0 + tid;
    unsigned long long word = 0ull;
    if (i < rhi) word = p.mask[((int64_t)h * T + start + i) * g.W + tile];
    const bool on = word != 0ull;
    const uint64_t bal = __ballot(on);
    if (lane == 0) Wcnt[wv] = __popcll(bal);
    __syncthreads();
    int before = 0, total = 0;
#pragma unroll
    for (int w = 0; w < NTH / 64; ++w) {
      before += w < wv ? Wcnt[w] : 0;
      total += Wcnt[w];
    }
    if (on) {
      const int at = before + __popcll(bal & ((1ull << lane) - 1ull));
      Rows[at] = i;
      Words[at] = word;
    }
    __syncthreads();
    for (int k = 0; k < NSR - 1 && k < total; ++k) issue(Rows[k], k);
    for (int k = 0; k < total; ++k) {
      // this wave's loads of row k have landed once at most the later rows'
      // loads are outstanding; the barrier then covers every wave's
      const int ahead = min(NSR - 2, total - 1 - k);
      if (ahead >= 2) wait_vm<2 * PER>();
      else if (ahead == 1) wait_vm<PER>();
      else wait_vm<0>();
      __syncthreads();
      if (k + NSR - 1 < total) issue(Rows[k + NSR - 1], (k + NSR - 1) % NSR);
      compute(k % NSR, Words[k]);
    }
    __syncthreads();  // the ring, Rows and Words are refilled
  }
  // lane (gq, r) holds dk_bar of chunks c0 + 16 wv + 4 gq + j, dims 16 nt + r
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    const int c = c0 + 16 * wv + 4 * gq + j;
    if (c < cs) {
      float* dst = p.dkb + ((kb0 + c) * g.Hkv + h) * (int64_t)D + r;
#pragma unroll
      for (int nt = 0; nt < NT; ++nt) atomicAdd(dst + 16 * nt, gs * acc[nt][j]);
    }
  }
}

// the summary's backward for one complete chunk and KV head
template <int D>
__global__ __launch_bounds__(256) void kbar_sum_bwd_kernel(Geom g, RouteBwdParams p) {
  constexpr int NTH = 256;
  __shared__ float Dkb[D];
  __shared__ float Qb[D];
  __shared__ float Pi[256], Dz[256];
  __shared__ float Red[NTH];
  const int c = blockIdx.x, s = blockIdx.y, h = blockIdx.z;
  const int tid = threadIdx.x;
  const SeqInfo si = seq_info(g.cu_seqlens, g.cu_chunks, s, g.max_seqlen, g.B);
  const int B = g.B;
  if ((c + 1) * B > si.len) return;   // complete chunks only
  const int64_t start = si.start;
  const int64_t kbrow = (si.chunk_off + c) * g.Hkv + h;
  for (int d = tid; d < D; d += NTH) {
    Dkb[d] = p.dkb[kbrow * D + d];
    Qb[d] = p.qbar[h * D + d];
  }
  __syncthreads();
  const float sD = 1.f / sqrtf((float)D);
  // thread t < B: key t's summary logit and <dk_bar, k_t>
  float z = -INFINITY, dpi = 0.f;
  if (tid < B) {
    const uint16_t* krow = (const uint16_t*)p.k + ((start + (int64_t)c * B + tid) * g.Hkv + h) * D;
    float a = 0.f, b = 0.f;
    for (int e = 0; e < D; e += 8) {
      const u32x4 kv = ldg16(krow + e);
#pragma unroll
      for (int w = 0; w < 4; ++w) {
        const float x0 = bf16lo(kv[w]), x1 = bf16hi(kv[w]);
        a = fmaf(x0, Qb[e + 2 * w], a);
        a = fmaf(x1, Qb[e + 2 * w + 1], a);
        b = fmaf(x0, Dkb[e + 2 * w], b);
        b = fmaf(x1, Dkb[e + 2 * w + 1], b);
      }
    }
    z = a * sD;
    dpi = b;
  }
  // softmax over the chunk's keys, block reductions through Red
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
  if (tid < B) {
    Pi[tid] = pi;
    Dz[tid] = pi * (dpi - pdp);
  }
  __syncthreads();
  // dk_t += pi_t dk_bar + sD dz_t q_bar (this chunk's rows of this head are
  // this workgroup's alone), coalesced over the dims
  for (int idx = tid; idx < B * D; idx += NTH) {
    const int t = idx / D, d = idx - (idx / D) * D;
    float* dk = p.dk + ((start + (int64_t)c * B + t) * g.Hkv + h) * D + d;
    *dk += Pi[t] * Dkb[d] + sD * Dz[t] * Qb[d];
  }
  // dq_bar += sD sum_t dz_t k_t
  for (int d = tid; d < D; d += NTH) {
    float t = 0.f;
    for (int kk = 0; kk < B; ++kk)
      t = fmaf(Dz[kk], bf16_to_f32(((const uint16_t*)p.k)[((start + (int64_t)c * B + kk) * g.Hkv + h) * D + d]), t);
    atomicAdd(&p.dqbar[h * D + d], sD * t);
  }
}

// The backward of every row's own-chunk estimate (k_hat_i = sum over the
// chunk's keys t <= i of pi_it k_t, pi_i = softmax(s <q_bar, k_t>) over those
// keys): one workgroup per chunk and KV head.  Row i's prefix softmax comes
// from the keys' logits z and its running max and sum; thread i forms
// dpi_it = <dk_hat_i, k_t> (dk_hat_i in registers), c_i = sum_t pi dpi and
// the column sums of dz_it = pi_it (dpi_it - c_i); then
// dk_t += sum_{i >= t} pi_it dk_hat_i + s colsum_t q_bar and
// dq_bar += s sum_t colsum_t k_t.
template <int D>
__global__ __launch_bounds__(256) void diag_sum_bwd_kernel(Geom g, RouteBwdParams p) {
  constexpr int NTH = 256;
  constexpr int KROW = D + 8;
  __shared__ __align__(16) uint16_t Ks[128 * KROW];
  __shared__ float Z[128], Mx[128], Sm[128], Cs[128], Qb[D];
  const int c = blockIdx.x, s = blockIdx.y, h = blockIdx.z;
  const int tid = threadIdx.x;
  const SeqInfo si = seq_info(g.cu_seqlens, g.cu_chunks, s, g.max_seqlen, g.B);
  const int B = g.B;
  const int r0 = c * B;
  if (c == 0 || r0 >= si.len) return;  // rows of a sequence's first chunk route nothing
  const int nr = min(B, si.len - r0);
  const int64_t tok0 = si.start + r0;
  const float sD = 1.f / sqrtf((float)D);
  // the chunk's keys (bf16, padded rows) and q_bar
  for (int idx = tid; idx < nr * (D / 8); idx += NTH) {
    const int t = idx / (D / 8), d0 = (idx % (D / 8)) * 8;
    *reinterpret_cast<u32x4*>(&Ks[t * KROW + d0]) =
        ldg16((const uint16_t*)p.k + ((tok0 + t) * g.Hkv + h) * (int64_t)D + d0);
  }
  for (int d = tid; d < D; d += NTH) Qb[d] = p.qbar[h * D + d];
  if (tid < 128) Cs[tid] = 0.f;
  __syncthreads();
  if (tid < nr) {
    float a = 0.f;
    for (int d = 0; d < D; ++d) a = fmaf(bf16_to_f32(Ks[tid * KROW + d]), Qb[d], a);
    Z[tid] = a * sD;
  }
  __syncthreads();
  // row i's running max and sum over keys t <= i
  if (tid < nr) {
    float m = -INFINITY;
    for (int t = 0; t <= tid; ++t) m = fmaxf(m, Z[t]);
    float sum = 0.f;
    for (int t = 0; t <= tid; ++t) sum += __expf(Z[t] - m);
    Mx[tid] = m;
    Sm[tid] = sum;
  }
  __syncthreads();
  if (tid < nr) {
    const int i = tid;
    float dkh[D];
    const float* src = p.dkdiag + ((tok0 + i) * g.Hkv + h) * (int64_t)D;
#pragma unroll
    for (int d = 0; d < D; d += 4) {
      const f32x4 v = *reinterpret_cast<const f32x4*>(src + d);
      dkh[d] = v[0];
      dkh[d + 1] = v[1];
      dkh[d + 2] = v[2];
      dkh[d + 3] = v[3];
    }
    const float m = Mx[i], inv = 1.f / Sm[i];
    // c_i = sum_t pi dpi, then the column sums of dz
    float ci = 0.f;
    for (int t = 0; t <= i; ++t) {
      float dp = 0.f;
#pragma unroll
      for (int d = 0; d < D; ++d) dp = fmaf(dkh[d], bf16_to_f32(Ks[t * KROW + d]), dp);
      ci = fmaf(__expf(Z[t] - m) * inv, dp, ci);
    }
    for (int t = 0; t <= i; ++t) {
      float dp = 0.f;
#pragma unroll
      for (int d = 0; d < D; ++d) dp = fmaf(dkh[d], bf16_to_f32(Ks[t * KROW + d]), dp);
      const float pi = __expf(Z[t] - m) * inv;
      atomicAdd(&Cs[t], pi * (dp - ci));
    }
  }
  __syncthreads();
  // dk_t += sum_{i >= t} pi_it dk_hat_i + s Cs_t q_bar: thread (t, d), d fastest
  for (int idx = tid; idx < nr * D; idx += NTH) {
    const int t = idx / D, d = idx - (idx / D) * D;
    float acc = sD * Cs[t] * Qb[d];
    for (int i = t; i < nr; ++i)
      acc = fmaf(__expf(Z[t] - Mx[i]) / Sm[i],
                 p.dkdiag[((tok0 + i) * g.Hkv + h) * (int64_t)D + d], acc);
    p.dk[((tok0 + t) * g.Hkv + h) * (int64_t)D + d] += acc;
  }
  // dq_bar += s sum_t Cs_t k_t
  for (int d = tid; d < D; d += NTH) {
    float acc = 0.f;
    for (int t = 0; t < nr; ++t) acc = fmaf(Cs[t], bf16_to_f32(Ks[t * KROW + d]), acc);
    atomicAdd(&p.dqbar[h * D + d], sD * acc);
  }
}

constexpr int kRbCap = 256;  // entries of route_bwd_kernel's first pass

int route_bwd_cpad(const Geom& g) { return ((g.max_seqlen / g.B) + 31) & ~31; }

hipError_t launch_route_bwd(const Geom& g, const RouteBwdParams& p, hipStream_t st) {
  if (g.T == 0) return hipSuccess;
  const int cs = g.max_seqlen / g.B;
  if (cs > 0) {
    const int64_t n = (int64_t)g.num_seqs * g.Hkv * g.D * p.cpad;
    hipLaunchKernelGGL(kbar_t_kernel, dim3((unsigned)((n + 255) / 256)), dim3(256), 0, st, g,
                       (const uint16_t*)p.kbar, const_cast<uint16_t*>(p.kbt), p.cpad);
  }
  // first pass: every row, the entries held for up to kRbCap chunks (the
  // active chunks of nearly every row: small LDS, many workgroups per CU);
  // the rows with more are flagged and take the wide pass, by range of
  // routable chunks for one sequence (a row at position i has floor(i/B) of
  // them, so the rows below CP*B fit the CP-wide variant), else all at once
  auto launch_rows = [&](int cp, int64_t lo, int64_t hi, int wide) {
    if (hi <= lo) return;
    dim3 grid((unsigned)(hi - lo), g.Hkv);
    const int r0 = (int)lo, r1 = (int)hi;
#define DASH_RB(DD, CPV) \
  hipLaunchKernelGGL((route_bwd_kernel<DD, CPV>), grid, dim3(256), 0, st, g, p, r0, r1, wide)
#define DASH_RB_CP(DD)                   \
  do {                                   \
    if (cp == 256) DASH_RB(DD, 256);     \
    else if (cp == 512) DASH_RB(DD, 512); \
    else if (cp == 1024) DASH_RB(DD, 1024); \
    else DASH_RB(DD, 2048);              \
  } while (0)
    if (g.D == 64) DASH_RB_CP(64); else DASH_RB_CP(128);
#undef DASH_RB_CP
#undef DASH_RB
  };
  launch_rows(kRbCap, 0, g.T, 0);
  const int cpmax = g.C_slots <= 512 ? 512 : g.C_slots <= 1024 ? 1024 : 2048;
  if (g.C_slots > kRbCap) {
    if (!g.cu_seqlens && g.num_seqs == 1) {
      for (int cp = cpmax; cp >= 512; cp /= 2) {
        const int64_t hi = std::min<int64_t>(g.T, (int64_t)cp * g.B);
        const int64_t lo = std::min<int64_t>(g.T, (int64_t)(cp / 2) * g.B);
        launch_rows(cp, lo, hi, 1);
      }
    } else {
      launch_rows(cpmax, 0, g.T, 1);
    }
  }
  if (cs == 0) return hipGetLastError();
  // chunk pass: 64-chunk tiles x row slices, about 2048 workgroups in all
  const int tiles = (cs + 63) / 64;
  const int base = tiles * g.num_seqs * g.Hkv;
  const int slices = std::max(1, std::min(g.max_seqlen / 256 + 1, (2048 + base - 1) / base));
  dim3 ggrid(tiles, slices, g.num_seqs * g.Hkv);
#define DASH_KG(DD, HH) hipLaunchKernelGGL((kbar_grad_kernel<DD, HH>), ggrid, dim3(256), 0, st, g, p)
  if (g.G == 16) {
    if (g.D == 64) DASH_KG(64, 1); else DASH_KG(128, 1);
  } else {
    if (g.D == 64) DASH_KG(64, 2); else DASH_KG(128, 2);
  }
#undef DASH_KG
  dim3 cgrid(cs, g.num_seqs, g.Hkv);
  if (g.D == 64)
    hipLaunchKernelGGL(kbar_sum_bwd_kernel<64>, cgrid, dim3(256), 0, st, g, p);
  else
    hipLaunchKernelGGL(kbar_sum_bwd_kernel<128>, cgrid, dim3(256), 0, st, g, p);
  if (p.kdiag) {
    // every chunk, the last partial one included
    dim3 dgrid((g.max_seqlen + g.B - 1) / g.B, g.num_seqs, g.Hkv);
    if (g.D == 64)
      hipLaunchKernelGGL(diag_sum_bwd_kernel<64>, dgrid, dim3(256), 0, st, g, p);
    else
      hipLaunchKernelGGL(diag_sum_bwd_kernel<128>, dgrid, dim3(256), 0, st, g, p);
  }
  return hipGetLastError();
}

}  // namespace dash
