// Phase 2, prefill: prior-induced sparse softmax attention ("Fase 2:
// Prior-Geinduceerde Spaarzame Softmax" of the gist.science technical summary:
// a FlashAttention-style loop over the active chunks of a bit-packed mask,
// the routing bias added to the logits before the softmax, and a separate
// diagonal branch for the query's own chunk).
//
// bf16 kernel.  A workgroup (8 waves) owns P consecutive positions of one
// chunk of one sequence for one KV head.  Its row tiles are 16 rows each
// (G query heads of 16/G positions, or 16 heads of one position), up to 16
// tiles, at most 2 per wave, with the online-softmax state of every tile in
// registers.
//   * The union of the P positions' active chunks is listed once in LDS; each
//     listed 64-key block of K and V is streamed from HBM once per workgroup,
//     through registers (prefetch of the next block while the current one is
//     consumed) into double-buffered LDS, V transposed.
//   * Each wave then runs every tile whose rows have that chunk active:
//     S^T = K Q^T with 16x16x32 bf16 MFMA (4 key tiles x D/32 steps), adds
//     s*<q,k>*log2(e) + log_prior*log2(e), updates the running max/sum in
//     base 2, and accumulates O^T += V^T P^T with the same MFMA.  Rows whose
//     position lacks the chunk get -inf; a tile with no such row skips it.
//   * The diagonal chunk follows with bias 0 and a causal mask.
// The score tiles come out with lane (g, r) holding row r and keys
// 16t + 4g + j, which is exactly the B operand layout of P^T for the PV MFMA
// when V^T's columns are stored in that order (attn_stage.h); the output
// O^T lands with lane (g, r) holding row r, so rescaling and normalising
// are per-lane.
//
// fp32 kernel (the small fp32 configurations): one wave per (token, query
// head) walking that row's own active chunks and diagonal with VALU math.
#include "attn_stage.h"
#include "dash_device.h"
#include "dash_internal.h"

namespace dash {

constexpr int kPrefillWaves = 8;
constexpr int kPrefillThreads = 64 * kPrefillWaves;
constexpr int kMaxTilesPerWave = 2;

struct TileGeom {
  int TP;             // positions per 16-row tile (G < 16)
  int HT;             // tiles per position (G >= 16)
  int NT;             // tiles per workgroup
  int TW;             // tiles per wave
  int P;              // positions per workgroup
  int tiles_per_seq;  // ceil(max_seqlen / P)
};

template <int D>
__global__ __launch_bounds__(kPrefillThreads, 1) void prefill_attn_bf16_kernel(
    Geom g, PrefillParams p, TileGeom tg) {
  constexpr int NTH = kPrefillThreads;
  constexpr int TWM = kMaxTilesPerWave;
  using C = StageCfg<D, NTH>;
  constexpr int KS = D / 32;
  constexpr int DT = D / 16;
  __shared__ __attribute__((aligned(16))) uint16_t Ks[2][C::KS_ELEMS];
  __shared__ __attribute__((aligned(16))) uint16_t Vt[2][C::VT_ELEMS];
  __shared__ unsigned long long Umask[32];
  __shared__ int Wpref[33];
  __shared__ uint16_t Blist[2048];

  const int tid = threadIdx.x, lane = tid & 63, wv = tid >> 6;
  const int r = lane & 15, gq = lane >> 4;
  const int tile = tg.tiles_per_seq - 1 - (int)blockIdx.x;  // longest rows first
  const int s = blockIdx.y, h = blockIdx.z;
  const SeqInfo si = seq_info(g.cu_seqlens, g.cu_chunks, s, g.max_seqlen, g.B);
  const int p0 = tile * tg.P;
  if (p0 >= si.len) return;
  const int pend = min(p0 + tg.P, si.len);
  const int cdiag = p0 / g.B;
  const int64_t T = g.T;
  const int W = g.W;
  const uint16_t* qp = (const uint16_t*)p.q;
  const uint16_t* kp = (const uint16_t*)p.k;
  const uint16_t* vp = (const uint16_t*)p.v;

  // ---- rows of this lane in each of the wave's tiles
  int rpos[TWM], rhead[TWM];
  bool rvalid[TWM], tvalid[TWM];
#pragma unroll
  for (int u = 0; u < TWM; ++u) {
    const int ti = wv * tg.TW + u;
    int pos, head;
    if (tg.TP == 1) {
      pos = p0 + ti / tg.HT;
      head = (ti % tg.HT) * 16 + r;
    } else {
      pos = p0 + ti * tg.TP + r / g.G;
      head = r % g.G;
    }
    rpos[u] = pos;
    rhead[u] = head;
    tvalid[u] = (u < tg.TW) && (ti < tg.NT);
    rvalid[u] = tvalid[u] && (pos < pend);
  }

  // ---- Q operands (B of S^T = K Q^T): lane (g, r) holds row r, dims 32ks + 8g ..
  bf16x8 qa[TWM][KS];
#pragma unroll
  for (int u = 0; u < TWM; ++u) {
    const int64_t qrow = ((si.start + rpos[u]) * g.Hq + h * g.G + rhead[u]) * (int64_t)D;
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) {
      u32x4 v = {0u, 0u, 0u, 0u};
      if (rvalid[u]) v = ldg16(qp + qrow + 32 * ks + 8 * gq);
      qa[u][ks] = as_bf16x8(v);
    }
  }

  // ---- union of the positions' active chunks -> ordered block list
  if (tid < 32) Umask[tid] = 0ull;
  __syncthreads();
  {
    const int npos = pend - p0;
    const unsigned long long* mbase =
        (const unsigned long long*)p.mask + ((int64_t)h * T + si.start + p0) * W;
    for (int idx = tid; idx < npos * W; idx += NTH) {
      const int w = idx % W;
      // only chunks before the workgroup's own chunk are routable
      const unsigned long long v = mbase[idx] & routable_bits(w, cdiag);
      if (v) atomicOr(&Umask[w], v);
    }
  }
  __syncthreads();
  if (tid < 64) {
    int cnt = (tid < W) ? __popcll(Umask[tid]) : 0;
    int inc = cnt;
#pragma unroll
    for (int o = 1; o < 64; o <<= 1) {
      const int y = __shfl_up(inc, o);
      if (lane >= o) inc += y;
    }
    if (tid < 33) Wpref[tid] = inc - cnt;  // exclusive prefix; Wpref[W] = total
  }
  __syncthreads();
  if (tid < W) {
    unsigned long long v = Umask[tid];
    int o = Wpref[tid];
    while (v) {
      Blist[o++] = (uint16_t)(tid * 64 + __ffsll(v) - 1);
      v &= v - 1;
    }
  }
  __syncthreads();
  const int SB = g.B / 64;
  const int nrouted = Wpref[W] * SB;
  const int ndiag = (pend - cdiag * g.B + 63) / 64;
  const int NS = nrouted + ndiag;

  // ---- per-tile state
  f32x4 o[TWM][DT];
  float m[TWM], l[TWM];
  unsigned long long mword[TWM];
  int mw_idx[TWM];
#pragma unroll
  for (int u = 0; u < TWM; ++u) {
    m[u] = -INFINITY;
    l[u] = 0.f;
    mword[u] = 0ull;
    mw_idx[u] = -1;
#pragma unroll
    for (int dt = 0; dt < DT; ++dt) o[u][dt] = f32x4{0.f, 0.f, 0.f, 0.f};
  }
  const float sl2 = p.scale * kLog2e;

  StageRegs<D, NTH> R;
  auto stage_key0 = [&](int st, int& c, bool& diag) -> int {
    if (st < nrouted) {
      c = Blist[st / SB];
      diag = false;
      return c * g.B + (st % SB) * 64;
    }
    c = cdiag;
    diag = true;
    return cdiag * g.B + (st - nrouted) * 64;
  };
  if (NS > 0) {
    int c0;
    bool d0;
    const int key0 = stage_key0(0, c0, d0);
    stage_load<D, NTH>(R, kp, vp, si.start, key0, d0 ? pend : si.len, g.Hkv, h, tid);
  }
  for (int st = 0; st < NS; ++st) {
    const int buf = st & 1;
    int c;
    bool diag;
    const int key0 = stage_key0(st, c, diag);
    stage_store<D, NTH>(R, Ks[buf], Vt[buf], tid);
    __syncthreads();
    if (st + 1 < NS) {
      int c1;
      bool d1;
      const int k1 = stage_key0(st + 1, c1, d1);
      stage_load<D, NTH>(R, kp, vp, si.start, k1, d1 ? pend : si.len, g.Hkv, h, tid);
    }
    const uint16_t* ks_ = Ks[buf];
    const uint16_t* vt_ = Vt[buf];
#pragma unroll
    for (int u = 0; u < TWM; ++u) {
      if (!tvalid[u]) break;
      bool rowon = rvalid[u];
      float bias = 0.f;
      if (!diag) {
        const int wi = c >> 6;
        if (wi != mw_idx[u]) {
          mw_idx[u] = wi;
          mword[u] = rvalid[u]
                         ? ((const unsigned long long*)p.mask)[((int64_t)h * T + si.start + rpos[u]) * W + wi]
                         : 0ull;
        }
        rowon = rowon && ((mword[u] >> (c & 63)) & 1ull);
        if (rowon)
          bias = p.log_prior[((int64_t)h * T + si.start + rpos[u]) * g.C_slots + c] * kLog2e;
      }
      if (__ballot(rowon) == 0ull) continue;
      // S^T tiles: sacc[t] lane (g, r) = score of row r, key 16t + 4g + j
      f32x4 sacc[4];
#pragma unroll
      for (int t = 0; t < 4; ++t) sacc[t] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int ks = 0; ks < KS; ++ks) {
#pragma unroll
        for (int t = 0; t < 4; ++t) {
          const bf16x8 ak = as_bf16x8(
              *reinterpret_cast<const u32x4*>(ks_ + (16 * t + r) * C::KSTR + 32 * ks + 8 * gq));
          sacc[t] = mfma16x16x32(ak, qa[u][ks], sacc[t]);
        }
      }
      float zmax = -INFINITY;
#pragma unroll
      for (int t = 0; t < 4; ++t) {
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          float z = sacc[t][j] * sl2 + bias;
          bool ok = rowon;
          if (diag) ok = ok && (key0 + 16 * t + 4 * gq + j <= rpos[u]);
          z = ok ? z : -INFINITY;
          sacc[t][j] = z;
          zmax = fmaxf(zmax, z);
        }
      }
      zmax = fmaxf(zmax, __shfl_xor(zmax, 16));
      zmax = fmaxf(zmax, __shfl_xor(zmax, 32));
      const float mnew = fmaxf(m[u], zmax);
      const float muse = (mnew == -INFINITY) ? 0.f : mnew;
      const float alpha = exp2f(m[u] - muse);
      float lsum = 0.f;
      uint32_t pk[4][2];
#pragma unroll
      for (int t = 0; t < 4; ++t) {
        const float p0_ = exp2f(sacc[t][0] - muse);
        const float p1_ = exp2f(sacc[t][1] - muse);
        const float p2_ = exp2f(sacc[t][2] - muse);
        const float p3_ = exp2f(sacc[t][3] - muse);
        lsum += (p0_ + p1_) + (p2_ + p3_);
        pk[t][0] = pack_bf16x2(p0_, p1_);
        pk[t][1] = pack_bf16x2(p2_, p3_);
      }
      l[u] = l[u] * alpha + lsum;
      m[u] = mnew;
#pragma unroll
      for (int dt = 0; dt < DT; ++dt) o[u][dt] *= alpha;
#pragma unroll
      for (int s2 = 0; s2 < 2; ++s2) {
        const u32x4 pb = {pk[2 * s2][0], pk[2 * s2][1], pk[2 * s2 + 1][0], pk[2 * s2 + 1][1]};
        const bf16x8 pbv = as_bf16x8(pb);
#pragma unroll
        for (int dt = 0; dt < DT; ++dt) {
          const bf16x8 av = as_bf16x8(
              *reinterpret_cast<const u32x4*>(vt_ + (16 * dt + r) * C::VSTR + 32 * s2 + 8 * gq));
          o[u][dt] = mfma16x16x32(av, pbv, o[u][dt]);
        }
      }
    }
  }

  // ---- epilogue: lane (g, r) holds row r, dims 16dt + 4g + j
#pragma unroll
  for (int u = 0; u < TWM; ++u) {
    if (!tvalid[u]) break;
    float lt = l[u];
    lt += __shfl_xor(lt, 16);
    lt += __shfl_xor(lt, 32);
    if (!rvalid[u]) continue;
    const float inv = 1.f / lt;
    const int64_t tok = si.start + rpos[u];
    uint16_t* orow = (uint16_t*)p.out + (tok * g.Hq + h * g.G + rhead[u]) * (int64_t)D;
#pragma unroll
    for (int dt = 0; dt < DT; ++dt) {
      const u32x2 w = {pack_bf16x2(o[u][dt][0] * inv, o[u][dt][1] * inv),
                       pack_bf16x2(o[u][dt][2] * inv, o[u][dt][3] * inv)};
      *reinterpret_cast<u32x2*>(orow + 16 * dt + 4 * gq) = w;
    }
    if (p.lse && gq == 0) {
      const float mu = (m[u] == -INFINITY) ? 0.f : m[u];
      p.lse[(int64_t)(h * g.G + rhead[u]) * T + tok] = (mu + __log2f(lt)) * kLn2;
    }
  }
}

// ---------------------------------------------------------------- fp32 rows

template <int D>
__global__ __launch_bounds__(64) void rowattn_f32_kernel(Geom g, PrefillParams p,
                                                         const int32_t* __restrict__ seqlens,
                                                         int64_t rows) {
  constexpr int DL = D / 64;  // output dims per lane
  __shared__ float qs[D];
  const int64_t row = blockIdx.x;
  const int qh = blockIdx.y;
  const int h = qh / g.G;
  const int lane = threadIdx.x;
  int64_t kbase;   // token row of the sequence's first key
  int pos;
  if (seqlens) {
    kbase = row * (int64_t)g.max_seqlen;
    pos = seqlens[row] - 1;
  } else {
    const int s = g.cu_seqlens ? find_seq(g.cu_seqlens, g.num_seqs, row)
                               : (int)(row / g.max_seqlen);
    const SeqInfo si = seq_info(g.cu_seqlens, g.cu_chunks, s, g.max_seqlen, g.B);
    kbase = si.start;
    pos = (int)(row - si.start);
  }
  const float* q = (const float*)p.q + (row * g.Hq + qh) * (int64_t)D;
  for (int d = lane; d < D; d += 64) qs[d] = q[d];
  __syncthreads();
  const float* kp = (const float*)p.k;
  const float* vp = (const float*)p.v;
  const float sl2 = p.scale * kLog2e;
  const unsigned long long* mrow =
      (const unsigned long long*)p.mask + ((int64_t)h * rows + row) * g.W;
  const float* lrow = p.log_prior + ((int64_t)h * rows + row) * g.C_slots;
  const int n = pos / g.B;
  float m = -INFINITY, l = 0.f, acc[DL];
#pragma unroll
  for (int e = 0; e < DL; ++e) acc[e] = 0.f;

  auto block = [&](int key0, int kend, float bias) {
    const int key = key0 + lane;
    float z = -INFINITY;
    if (key < kend) {
      const float* kr = kp + ((kbase + key) * g.Hkv + h) * (int64_t)D;
      float d = 0.f;
      for (int e = 0; e < D; e += 4) {
        const f32x4 k4 = *reinterpret_cast<const f32x4*>(kr + e);
        d = fmaf(qs[e], k4[0], d);
        d = fmaf(qs[e + 1], k4[1], d);
        d = fmaf(qs[e + 2], k4[2], d);
        d = fmaf(qs[e + 3], k4[3], d);
      }
      z = d * sl2 + bias;
    }
    const float mx = wave_max(z);
    const float mnew = fmaxf(m, mx);
    const float muse = (mnew == -INFINITY) ? 0.f : mnew;
    const float a = exp2f(m - muse);
    const float pz = exp2f(z - muse);
    l = l * a + wave_sum(pz);
    m = mnew;
#pragma unroll
    for (int e = 0; e < DL; ++e) acc[e] *= a;
    const int nk = min(64, kend - key0);
    for (int j = 0; j < nk; ++j) {
      const float pj = __shfl(pz, j);
      const float* vr = vp + ((kbase + key0 + j) * g.Hkv + h) * (int64_t)D;
#pragma unroll
      for (int e = 0; e < DL; ++e) acc[e] = fmaf(pj, vr[lane + 64 * e], acc[e]);
    }
  };
  for (int w = 0; w * 64 < n; ++w) {
    unsigned long long bits = mrow[w] & routable_bits(w, n);
    while (bits) {
      const int c = w * 64 + __ffsll(bits) - 1;
      bits &= bits - 1;
      const float bias = lrow[c] * kLog2e;
      for (int sb = 0; sb < g.B; sb += 64) block(c * g.B + sb, c * g.B + sb + 64, bias);
    }
  }
  for (int key0 = n * g.B; key0 <= pos; key0 += 64) block(key0, pos + 1, 0.f);
  const float inv = 1.f / l;
  float* orow = (float*)p.out + (row * g.Hq + qh) * (int64_t)D;
#pragma unroll
  for (int e = 0; e < DL; ++e) orow[lane + 64 * e] = acc[e] * inv;
  if (p.lse && lane == 0) p.lse[(int64_t)qh * rows + row] = (m + __log2f(l)) * kLn2;
}

// Up to 16 tiles per workgroup, never more positions than one chunk.
static TileGeom make_tiles(const Geom& g) {
  TileGeom t;
  t.TP = g.G >= 16 ? 1 : 16 / g.G;
  t.HT = g.G >= 16 ? g.G / 16 : 1;
  t.NT = min(kPrefillWaves * kMaxTilesPerWave, g.B * t.HT / t.TP);
  t.TW = (t.NT + kPrefillWaves - 1) / kPrefillWaves;
  t.P = t.NT * t.TP / t.HT;
  t.tiles_per_seq = (g.max_seqlen + t.P - 1) / t.P;
  return t;
}

hipError_t launch_prefill_attn(const Geom& g, const PrefillParams& p, hipStream_t st) {
  if (g.T == 0) return hipSuccess;
  if (g.bf16) {
    const TileGeom tg = make_tiles(g);
    dim3 grid(tg.tiles_per_seq, g.num_seqs, g.Hkv);
    if (g.D == 64)
      hipLaunchKernelGGL(prefill_attn_bf16_kernel<64>, grid, dim3(kPrefillThreads), 0, st, g,
                         p, tg);
    else
      hipLaunchKernelGGL(prefill_attn_bf16_kernel<128>, grid, dim3(kPrefillThreads), 0, st, g,
                         p, tg);
  } else {
    dim3 grid((unsigned)g.T, g.Hq);
    if (g.D == 64)
      hipLaunchKernelGGL(rowattn_f32_kernel<64>, grid, dim3(64), 0, st, g, p, nullptr, g.T);
    else
      hipLaunchKernelGGL(rowattn_f32_kernel<128>, grid, dim3(64), 0, st, g, p, nullptr, g.T);
  }
  return hipGetLastError();
}

// fp32 decode rows reuse the row kernel (declared for attn_decode.hip).
hipError_t launch_rowattn_f32_decode(const Geom& g, const PrefillParams& p,
                                     const int32_t* seqlens, int64_t batch, hipStream_t st) {
  dim3 grid((unsigned)batch, g.Hq);
  if (g.D == 64)
    hipLaunchKernelGGL(rowattn_f32_kernel<64>, grid, dim3(64), 0, st, g, p, seqlens, batch);
  else
    hipLaunchKernelGGL(rowattn_f32_kernel<128>, grid, dim3(64), 0, st, g, p, seqlens, batch);
  return hipGetLastError();
}

}  // namespace dash
