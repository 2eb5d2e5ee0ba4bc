// Phase 2, prefill: prior-induced sparse softmax attention ("Fase 2:
// Prior-Geinduceerde Spaarzame Softmax" of the gist.science technical summary:
// a FlashAttention-style loop over the active chunks of a bit-packed mask,
// the routing bias added to the logits before the softmax, and a separate
// diagonal branch for the query's own chunk).
//
// Three kernels:
//   * prefill_attn_ring_kernel (bf16, GQA group G >= 16): a 16-row MFMA tile
//     is the 16 query heads of one position, so tiles share their mask.  A
//     workgroup of 8 waves owns 16 tiles (two per wave) and streams the union
//     of its positions' active chunks, then its diagonal blocks, through a
//     4-slot LDS ring filled by direct global->LDS loads of K rows and of a
//     transposed V (vt_transpose_kernel writes V^T first).  A per-chunk
//     activity bitmap built up front tells each wave which of its tiles visit
//     a staged block.  See the comments at the kernel for the details.
//   * prefill_attn_bf16_kernel (bf16, G < 16): 16-row tiles of G heads x 16/G
//     positions; K and V staged through registers into double-buffered LDS.
//   * rowattn_f32_kernel (fp32): one wave per (token, query head) walking the
//     row's own active chunks and diagonal with VALU math.
// Every visit of a 16-row tile to a 64-key block computes S^T = K Q^T with
// 16x16x32 bf16 MFMA, adds s*<q,k>*log2(e) + log_prior*log2(e), updates the
// running max/sum in base 2, and accumulates O^T += V^T P^T with the same
// MFMA.  The score tiles come out with lane (g, r) holding row r and keys
// 16t + 4g + j, which is exactly the B operand layout of P^T for the PV
// MFMA when V^T's columns are stored in that order (attn_stage.h); O^T lands
// with lane (g, r) holding row r, so rescaling and normalising are per-lane.
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

// Reference-point slack of the running maximum (log2 units): a row's
// exponent offset is only moved when its maximum grows by more than this, so
// the accumulators are rescaled rarely; p = exp2(z - m) then stays <= 2^8.
constexpr float kRescale = 8.f;

// One visit: a 16-row tile against one staged 64-key block.
//   MASKED = false: every row of the tile attends every key of the block.
//   MASKED = true : row r attends key j iff rowon and (!diag or j <= rpos).
template <int D, bool MASKED>
__device__ __forceinline__ void visit(const uint16_t* __restrict__ ks_,
                                      const uint16_t* __restrict__ vt_, int koff, int voff,
                                      const bf16x8 (&qa)[D / 32], f32x4 (&o)[D / 16],
                                      f32x4& lacc, float& m, float sl2, float bz, bool rowon,
                                      bool diag, int kbase, int rpos) {
  using C = StageCfg<D, kPrefillThreads>;
  constexpr int KS = D / 32;
  constexpr int DT = D / 16;
  // S^T = K Q^T: sacc[t] lane (g, r) = raw score of row r, key 16t + 4g + j
  f32x4 sacc[4];
#pragma unroll
  for (int t = 0; t < 4; ++t) sacc[t] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
  for (int ks = 0; ks < KS; ++ks) {
#pragma unroll
    for (int t = 0; t < 4; ++t) {
      const bf16x8 ak = as_bf16x8(
          *reinterpret_cast<const u32x4*>(ks_ + koff + 16 * t * C::KSTR + 32 * ks));
      sacc[t] = mfma16x16x32(ak, qa[ks], sacc[t]);
    }
  }
  bool ok[4][4];
  float amax = -INFINITY;
  if constexpr (MASKED) {
#pragma unroll
    for (int t = 0; t < 4; ++t)
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        ok[t][j] = rowon && (!diag || kbase + 16 * t + j <= rpos);
        amax = fmaxf(amax, ok[t][j] ? sacc[t][j] : -INFINITY);
      }
  } else {
#pragma unroll
    for (int t = 0; t < 4; ++t)
      amax = fmaxf(amax, fmaxf(fmaxf(sacc[t][0], sacc[t][1]), fmaxf(sacc[t][2], sacc[t][3])));
  }
  amax = fmaxf(amax, xor16(amax));
  amax = fmaxf(amax, xor32(amax));
  // scale > 0, so the largest logit of the row is amax * scale + bias
  const float zmax = amax * sl2 + bz;
  const bool up = zmax > m + kRescale;
  if (__ballot(up) != 0ull) {
    const float mn = up ? zmax : m;
    const float alpha = up ? exp2f(m - mn) : 1.f;
#pragma unroll
    for (int dt = 0; dt < DT; ++dt) o[dt] *= alpha;
    lacc *= alpha;
    m = mn;
  }
  const float off = bz - m;
  uint32_t pk[4][2];
#pragma unroll
  for (int t = 0; t < 4; ++t) {
    float pv[4];
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      pv[j] = __builtin_amdgcn_exp2f(fmaf(sacc[t][j], sl2, off));
      if constexpr (MASKED) pv[j] = ok[t][j] ? pv[j] : 0.f;
    }
    pk[t][0] = cvt_pk_bf16(pv[0], pv[1]);
    pk[t][1] = cvt_pk_bf16(pv[2], pv[3]);
  }
  // O^T += V^T P^T and, with an all-ones A operand, the row sums of P
  const u32x4 ones_u = {0x3f803f80u, 0x3f803f80u, 0x3f803f80u, 0x3f803f80u};
  const bf16x8 ones = as_bf16x8(ones_u);
#pragma unroll
  for (int s2 = 0; s2 < 2; ++s2) {
    const u32x4 pb = {pk[2 * s2][0], pk[2 * s2][1], pk[2 * s2 + 1][0], pk[2 * s2 + 1][1]};
    const bf16x8 pbv = as_bf16x8(pb);
#pragma unroll
    for (int dt = 0; dt < DT; ++dt) {
      const bf16x8 av = as_bf16x8(
          *reinterpret_cast<const u32x4*>(vt_ + voff + 16 * dt * C::VSTR + 32 * s2));
      o[dt] = mfma16x16x32(av, pbv, o[dt]);
    }
    lacc = mfma16x16x32(ones, pbv, lacc);
  }
}

template <int D, bool UNI>
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
  const unsigned long long* mask = (const unsigned long long*)p.mask;

  // ---- rows of this lane in each of the wave's tiles (UNI: one position per tile)
  int rpos[TWM], rhead[TWM];
  bool rvalid[TWM], tvalid[TWM];
#pragma unroll
  for (int u = 0; u < TWM; ++u) {
    const int ti = wv * tg.TW + u;
    int pos, head;
    if (UNI) {
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
    const unsigned long long* mbase = mask + ((int64_t)h * T + si.start + p0) * W;
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

  // ---- per-tile state: O^T (lane (g, r): row r, dims 16dt + 4g + j), row sums, offsets
  f32x4 o[TWM][DT];
  f32x4 lacc[TWM];
  float m[TWM];
  unsigned long long mword[TWM];
  int mw_idx[TWM];
  int64_t prow[TWM];  // token row of the tile's position (UNI) / of this lane's row
#pragma unroll
  for (int u = 0; u < TWM; ++u) {
    m[u] = -INFINITY;
    lacc[u] = f32x4{0.f, 0.f, 0.f, 0.f};
    mword[u] = 0ull;
    mw_idx[u] = -1;
    prow[u] = (int64_t)h * T + si.start + min(rpos[u], pend - 1);
    if (UNI) prow[u] = uniform64(prow[u]);
#pragma unroll
    for (int dt = 0; dt < DT; ++dt) o[u][dt] = f32x4{0.f, 0.f, 0.f, 0.f};
  }
  const float sl2 = p.scale * kLog2e;
  const int koff = r * C::KSTR + 8 * gq;
  const int voff = r * C::VSTR + 8 * gq;

  Stager<D, NTH> stg((const uint16_t*)p.k, (const uint16_t*)p.v, si.start, g.Hkv, h, tid);
  StageRegs<D, NTH> R;
  auto stage_key0 = [&](int st, int& c) -> int {
    if (st < nrouted) {
      c = Blist[st / SB];
      return c * g.B + (st % SB) * 64;
    }
    c = cdiag;
    return cdiag * g.B + (st - nrouted) * 64;
  };
  if (NS > 0) {
    int c0;
    const int key0 = stage_key0(0, c0);
    if (nrouted > 0) stg.load(R, key0); else stg.load_guarded(R, key0, pend);
  }
  for (int st = 0; st < NS; ++st) {
    const int buf = st & 1;
    int c;
    const int key0 = stage_key0(st, c);
    const bool diag = st >= nrouted;
    stage_store<D, NTH>(R, Ks[buf], Vt[buf], tid);
    __syncthreads();
    if (st + 1 < NS) {
      int c1;
      const int k1 = stage_key0(st + 1, c1);
      if (st + 1 < nrouted) stg.load(R, k1); else stg.load_guarded(R, k1, pend);
    }
    const uint16_t* ks_ = Ks[buf];
    const uint16_t* vt_ = Vt[buf];
#pragma unroll
    for (int u = 0; u < TWM; ++u) {
      if (!tvalid[u]) break;
      if (!diag) {
        const int wi = c >> 6;
        if (wi != mw_idx[u]) {
          mw_idx[u] = wi;
          mword[u] = mask[prow[u] * W + wi];
        }
        const bool rowon = rvalid[u] && ((mword[u] >> (c & 63)) & 1ull);
        if (UNI) {
          if (!rowon) continue;  // wave-uniform: the whole tile is one position
          const float bz = p.log_prior[prow[u] * g.C_slots + c] * kLog2e;
          visit<D, false>(ks_, vt_, koff, voff, qa[u], o[u], lacc[u], m[u], sl2, bz, true,
                          false, 0, 0);
        } else {
          if (__ballot(rowon) == 0ull) continue;
          const float bz = rowon ? p.log_prior[prow[u] * g.C_slots + c] * kLog2e : 0.f;
          visit<D, true>(ks_, vt_, koff, voff, qa[u], o[u], lacc[u], m[u], sl2, bz, rowon,
                         false, 0, 0);
        }
      } else {
        if (__ballot(rvalid[u]) == 0ull) continue;
        visit<D, true>(ks_, vt_, koff, voff, qa[u], o[u], lacc[u], m[u], sl2, 0.f, rvalid[u],
                       true, key0 + 4 * gq, rpos[u]);
      }
    }
  }

  // ---- epilogue: normalise by the row sums (lacc holds the full sum of row r)
#pragma unroll
  for (int u = 0; u < TWM; ++u) {
    if (!tvalid[u]) break;
    if (!rvalid[u]) continue;
    const float lt = lacc[u][0];
    const float inv = 1.f / lt;
    const int64_t tok = si.start + rpos[u];
    uint16_t* orow = (uint16_t*)p.out + (tok * g.Hq + h * g.G + rhead[u]) * (int64_t)D;
#pragma unroll
    for (int dt = 0; dt < DT; ++dt) {
      const u32x2 w = {cvt_pk_bf16(o[u][dt][0] * inv, o[u][dt][1] * inv),
                       cvt_pk_bf16(o[u][dt][2] * inv, o[u][dt][3] * inv)};
      *reinterpret_cast<u32x2*>(orow + 16 * dt + 4 * gq) = w;
    }
    if (p.lse && gq == 0)
      p.lse[(int64_t)(h * g.G + rhead[u]) * T + tok] = (m[u] + __log2f(lt)) * kLn2;
  }
}

// ---------------------------------------------------------------- V^T + ring

// First padded column of sequence s in V^T.
__device__ __forceinline__ int64_t pad_off(const Geom& g, int s) {
  return g.cu_seqlens ? (int64_t)g.cu_pad[s] : (int64_t)s * ((g.max_seqlen + 63) / 64 * 64);
}

// V^T[h][d][pad_off(s) + 64 kb + vt_col(j)] = v[start + 64 kb + j][h][d], zero
// past the sequence end: the PV operand layout, so the attention kernel can
// copy 128-byte rows of it straight into LDS.  One workgroup per
// (64-key block, sequence, KV head).
template <int D>
__global__ __launch_bounds__(256) void vt_transpose_kernel(Geom g, const uint16_t* __restrict__ v,
                                                           uint16_t* __restrict__ vt,
                                                           int64_t Tp) {
  constexpr int KPT = D / 32;           // keys per thread (4 or 2)
  constexpr int NKG = 64 / KPT;
  const int kb = blockIdx.x, s = blockIdx.y, h = blockIdx.z;
  const SeqInfo si = seq_info(g.cu_seqlens, nullptr, s, g.max_seqlen, g.B);
  if (kb * 64 >= si.len) return;
  const int tid = threadIdx.x;
  const int kg = tid % NKG, vpiece = tid / NKG;
  u32x4 x[KPT];
#pragma unroll
  for (int i = 0; i < KPT; ++i) {
    const int key = kb * 64 + kg * KPT + i;
    u32x4 z = {0u, 0u, 0u, 0u};
    if (key < si.len) z = ldg16(v + ((si.start + key) * g.Hkv + h) * (int64_t)D + vpiece * 8);
    x[i] = z;
  }
  const int64_t col = pad_off(g, s) + kb * 64 + vt_col(kg * KPT);
  uint16_t* base = vt + ((int64_t)h * D + vpiece * 8) * Tp + col;
#pragma unroll
  for (int w = 0; w < 4; ++w) {
    if constexpr (KPT == 4) {
      const u32x2 lo = {__builtin_amdgcn_perm(x[1][w], x[0][w], 0x05040100u),
                        __builtin_amdgcn_perm(x[3][w], x[2][w], 0x05040100u)};
      const u32x2 hi = {__builtin_amdgcn_perm(x[1][w], x[0][w], 0x07060302u),
                        __builtin_amdgcn_perm(x[3][w], x[2][w], 0x07060302u)};
      *reinterpret_cast<u32x2*>(base + (2 * w) * Tp) = lo;
      *reinterpret_cast<u32x2*>(base + (2 * w + 1) * Tp) = hi;
    } else {
      *reinterpret_cast<uint32_t*>(base + (2 * w) * Tp) =
          __builtin_amdgcn_perm(x[1][w], x[0][w], 0x05040100u);
      *reinterpret_cast<uint32_t*>(base + (2 * w + 1) * Tp) =
          __builtin_amdgcn_perm(x[1][w], x[0][w], 0x07060302u);
    }
  }
}

constexpr int kRing = 4;       // LDS slots; up to 3 blocks in flight
constexpr int kRingWaves = 8;  // two 16-row tiles per wave
constexpr int kRingThreads = 64 * kRingWaves;
constexpr int kRingTiles = 2 * kRingWaves;

template <int D>
struct RingCfg {
  static constexpr int KROW = D * 2;                  // bytes per K row
  static constexpr int KP = KROW / 16;                // 16-byte pieces per K row
  static constexpr int KBYTES = 64 * KROW;
  static constexpr int VROW = 128;                    // bytes per V^T row (64 keys)
  static constexpr int VBYTES = D * VROW;
  static constexpr int STAGE = KBYTES + VBYTES;
  static constexpr int NP = STAGE / (16 * kRingThreads);  // 16-byte loads per thread
  static constexpr int LPS = NP + 1;                      // + the tiles' bias words
  static_assert(NP * 16 * kRingThreads == STAGE, "slot must split into whole loads");
  static_assert(KBYTES % (NP * 1024) == 0, "a wave's pieces lie all in K or all in V^T");
};

// XOR swizzle of the 16-byte pieces of an LDS row: 16 consecutive rows read
// at one logical piece land in 16 different 4-bank groups.
template <int P>
__device__ __forceinline__ int swz(int row) {
  return P == 16 ? (row & 15) : ((row >> 1) & 7);
}

// One visit of tiles U0 .. U0+NTL-1 of a wave (16 rows each) to one staged
// 64-key block (ring layout): S^T = K Q^T, online softmax in base 2 with the
// tile's bias for the block, O^T += V^T P^T.  With two tiles, every K and V^T
// fragment read from LDS feeds both tiles' MFMAs.
// The row sum l is accumulated from the same bf16-rounded P that enters the
// PV product (v_dot2 against (1, 1)); lane (g, r) holds the partial sum of
// row r over its keys 16t + 4g + j, the four partials are added at the end.
//   MASKED = false: every row attends every key of the block.
//   MASKED = true : a row attends key j iff key index <= its position.
// LDS fragments are read in groups of four 16-byte loads, two groups ahead of
// the MFMAs that consume them (sched_barrier keeps the compiler from
// collapsing the pipeline); the first two V^T groups are read during the
// softmax, which does not need them.
template <int D, bool MASKED, int U0, int NTL>
__device__ __forceinline__ void visit_ring(lds_u8* ks_, lds_u8* vt_,
                                           const int (&koff)[D / 32], const int (&voff)[2],
                                           const bf16x8 (&qa)[2][D / 32], f32x4 (&o)[2][D / 16],
                                           float (&l)[2], float (&m)[2], float sl2,
                                           const float (&bz)[2], int kbase, const int (&rpos)[2]) {
  using R = RingCfg<D>;
  constexpr int KS = D / 32;
  constexpr int DT = D / 16;
  constexpr int NVG = 2 * DT / 4;  // V^T groups of four fragments
  auto kload = [&](u32x4 (&f)[4], int ks) {
#pragma unroll
    for (int t = 0; t < 4; ++t)
      f[t] = lds_read16(ks_ + koff[ks] + 16 * t * R::KROW);
  };
  // group vg covers s2 = vg / (DT / 4), dt = 4 (vg % (DT / 4)) .. +3
  auto vload = [&](u32x4 (&f)[4], int vg) {
    const int s2 = vg / (DT / 4), dt0 = 4 * (vg % (DT / 4));
#pragma unroll
    for (int i = 0; i < 4; ++i)
      f[i] = lds_read16(vt_ + voff[s2] + 16 * (dt0 + i) * R::VROW);
  };
  // fragment groups 0 .. KS-1 are K (ks = g), KS .. KS+NVG-1 are V^T; three
  // buffers, two groups in flight ahead of the one being consumed
  constexpr int NG = KS + NVG;
  u32x4 fr[3][4];
  auto gload = [&](int gi) {
    if (gi < KS) kload(fr[gi % 3], gi);
    else if (gi < NG) vload(fr[gi % 3], gi - KS);
  };
  f32x4 sacc[NTL][4];
#pragma unroll
  for (int u = 0; u < NTL; ++u)
#pragma unroll
    for (int t = 0; t < 4; ++t) sacc[u][t] = f32x4{0.f, 0.f, 0.f, 0.f};
  gload(0);
  gload(1);
#pragma unroll
  for (int ks = 0; ks < KS; ++ks) {
    gload(ks + 2);
    __builtin_amdgcn_sched_barrier(0);
#pragma unroll
    for (int t = 0; t < 4; ++t)
#pragma unroll
      for (int u = 0; u < NTL; ++u)
        sacc[u][t] = mfma16x16x32(as_bf16x8(fr[ks % 3][t]), qa[U0 + u][ks], sacc[u][t]);
    __builtin_amdgcn_sched_barrier(0);
  }
  uint32_t pk[NTL][4][2];
#pragma unroll
  for (int u = 0; u < NTL; ++u) {
    // causal mask folded into the scores: keys past the row's position get
    // -inf here and p = 0 below (no per-element mask outlives its compare)
    if constexpr (MASKED) {
#pragma unroll
      for (int t = 0; t < 4; ++t)
#pragma unroll
        for (int j = 0; j < 4; ++j)
          sacc[u][t][j] = kbase + 16 * t + j <= rpos[U0 + u] ? sacc[u][t][j] : -INFINITY;
    }
    float amax = -INFINITY;
#pragma unroll
    for (int t = 0; t < 4; ++t)
      amax = fmaxf(amax, fmaxf(fmaxf(sacc[u][t][0], sacc[u][t][1]),
                               fmaxf(sacc[u][t][2], sacc[u][t][3])));
    amax = fmaxf(amax, xor16(amax));
    amax = fmaxf(amax, xor32(amax));
    const float zmax = amax * sl2 + bz[U0 + u];
    float& mu = m[U0 + u];
    const bool up = zmax > mu + kRescale;
    if (__ballot(up) != 0ull) {
      const float mn = up ? zmax : mu;
      const float alpha = up ? exp2f(mu - mn) : 1.f;
#pragma unroll
      for (int dt = 0; dt < DT; ++dt) o[U0 + u][dt] *= alpha;
      l[U0 + u] *= alpha;
      mu = mn;
    }
    const float off = bz[U0 + u] - mu;
#pragma unroll
    for (int t = 0; t < 4; ++t) {
      float pv[4];
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        pv[j] = __builtin_amdgcn_exp2f(fmaf(sacc[u][t][j], sl2, off));
        if constexpr (MASKED) pv[j] = sacc[u][t][j] == -INFINITY ? 0.f : pv[j];
      }
      pk[u][t][0] = cvt_pk_bf16(pv[0], pv[1]);
      pk[u][t][1] = cvt_pk_bf16(pv[2], pv[3]);
    }
    float la = l[U0 + u], lb = 0.f;
#pragma unroll
    for (int t = 0; t < 4; ++t) {
      la = dot2_bf16_ones(pk[u][t][0], la);
      lb = dot2_bf16_ones(pk[u][t][1], lb);
    }
    l[U0 + u] = la + lb;
  }
  __builtin_amdgcn_sched_barrier(0);
#pragma unroll
  for (int vg = 0; vg < NVG; ++vg) {
    gload(KS + vg + 2);
    __builtin_amdgcn_sched_barrier(0);
    const int s2 = vg / (DT / 4), dt0 = 4 * (vg % (DT / 4));
    u32x4 (&cur)[4] = fr[(KS + vg) % 3];
#pragma unroll
    for (int u = 0; u < NTL; ++u) {
      const u32x4 pb = {pk[u][2 * s2][0], pk[u][2 * s2][1], pk[u][2 * s2 + 1][0],
                        pk[u][2 * s2 + 1][1]};
#pragma unroll
      for (int i = 0; i < 4; ++i)
        o[U0 + u][dt0 + i] =
            mfma16x16x32(as_bf16x8(cur[i]), as_bf16x8(pb), o[U0 + u][dt0 + i]);
    }
    __builtin_amdgcn_sched_barrier(0);
  }
}

// Prefill attention for G >= 16 (every 16-row tile is 16 query heads of one
// position; 16 tiles per workgroup, two per wave).  The blocks of the
// workgroup's list stream through a 4-slot LDS ring filled by direct
// global->LDS loads (K rows from K, V^T rows from the V^T workspace, and each
// tile's bias for the block), three blocks ahead of the one being consumed.
// Which positions have each listed chunk active is worked out once, up front,
// into a bitmap in LDS, so the loop reads no memory but LDS.  A wave visits a
// block with both its tiles at once when both have it active.  The loop is
// unrolled by the ring depth so every slot is a distinct LDS array; waits are
// counted (vmcnt) and the barrier carries no fence.
template <int D>
__global__ __launch_bounds__(kRingThreads, 1) void prefill_attn_ring_kernel(
    Geom g, PrefillParams p, TileGeom tg) {
  constexpr int NTH = kRingThreads;
  using R = RingCfg<D>;
  constexpr int KS = D / 32;
  constexpr int DT = D / 16;
  __shared__ __attribute__((aligned(1024))) uint8_t ring[kRing][R::STAGE];
  __shared__ float bias[kRing][kRingTiles];
  __shared__ unsigned long long Umask[32];
  __shared__ int Wpref[33];
  __shared__ uint16_t Blist[2048];
  __shared__ uint16_t Act[2048];   // bit t: position p0 + t has chunk Blist[j] active

  const int tid = threadIdx.x, lane = tid & 63;
  const int wv = __builtin_amdgcn_readfirstlane(tid >> 6);  // wave index, held in an SGPR
  const int r = lane & 15, gq = lane >> 4;
  const int tile = tg.tiles_per_seq - 1 - (int)blockIdx.x;
  const int s = blockIdx.y, h = blockIdx.z;
  const SeqInfo si = seq_info(g.cu_seqlens, nullptr, s, g.max_seqlen, g.B);
  const int p0 = tile * tg.P;
  if (p0 >= si.len) return;
  const int pend = min(p0 + tg.P, si.len);
  const int npos = pend - p0;
  const int cdiag = p0 / g.B;
  const int64_t T = g.T;
  const int W = g.W;
  const unsigned long long* __restrict__ mask = (const unsigned long long*)p.mask;

  // this wave's tiles u = 0, 1: 16 heads (rhead) of position rpos = p0 + tpos
  int tpos[2], rpos[2], rhead[2];
  bool rvalid[2];
#pragma unroll
  for (int u = 0; u < 2; ++u) {
    const int ti = 2 * wv + u;
    tpos[u] = ti / tg.HT;
    rpos[u] = p0 + tpos[u];
    rhead[u] = (ti % tg.HT) * 16 + r;
    rvalid[u] = rpos[u] < pend;
  }
  bf16x8 qa[2][KS];
#pragma unroll
  for (int u = 0; u < 2; ++u) {
    const int64_t qrow = ((si.start + rpos[u]) * g.Hq + h * g.G + rhead[u]) * (int64_t)D;
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) {
      u32x4 v = {0u, 0u, 0u, 0u};
      if (rvalid[u]) v = ldg16((const uint16_t*)p.q + qrow + 32 * ks + 8 * gq);
      qa[u][ks] = as_bf16x8(v);
    }
  }

  // ---- ordered list of the union of the positions' active chunks, and for
  // each listed chunk the positions that have it active
  if (tid < 32) Umask[tid] = 0ull;
  __syncthreads();
  const unsigned long long* mbase = mask + ((int64_t)h * T + si.start + p0) * W;
  for (int idx = tid; idx < npos * W; idx += NTH) {
    const int w = idx % W;
    const unsigned long long v = mbase[idx] & routable_bits(w, cdiag);
    if (v) atomicOr(&Umask[w], v);
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
    if (tid < 33) Wpref[tid] = inc - cnt;
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
  const int nlist = Wpref[W];
  for (int j = tid; j < nlist; j += NTH) {
    const int c = Blist[j];
    uint32_t bits = 0;
    for (int t = 0; t < npos; ++t)
      bits |= (uint32_t)((mbase[t * W + (c >> 6)] >> (c & 63)) & 1ull) << t;
    Act[j] = (uint16_t)bits;
  }
  __syncthreads();
  const int sbl = g.B == 128 ? 1 : 0;  // log2 of the 64-key blocks per chunk
  const int nrouted = nlist << sbl;
  const int ndiag = (pend - cdiag * g.B + 63) / 64;
  const int NS = nrouted + ndiag;

  // ---- per-thread DMA sources (piece layout fixed per thread; a wave's
  // pieces are all K rows or all V^T rows)
  const int64_t krs = (int64_t)g.Hkv * D * 2;  // bytes between consecutive keys
  const int64_t vrs = p.Tp * 2;                  // bytes between V^T rows
  const bool isk = wv * R::NP * 1024 < R::KBYTES;
  const uint8_t* kbase = (const uint8_t*)p.k + (si.start * (int64_t)g.Hkv + h) * D * 2;
  const uint8_t* vbase = (const uint8_t*)p.vt + ((int64_t)h * D * p.Tp + pad_off(g, s)) * 2;
  // piece i of this thread: K row or V^T row kr[i] of the block, at source
  // address pbase[i] + (K: key0 * krs, V^T: key0 * 2) for the block at key0
  const uint8_t* pbase[R::NP];
  int kr[R::NP];
#pragma unroll
  for (int i = 0; i < R::NP; ++i) {
    const int o = (wv * R::NP + i) * 1024 + lane * 16;
    if (isk) {
      kr[i] = o / R::KROW;
      const int pcol = (((o % R::KROW) / 16) ^ swz<R::KP>(kr[i])) * 16;
      pbase[i] = kbase + kr[i] * krs + pcol;
    } else {
      const int ov = o - R::KBYTES;
      kr[i] = ov / R::VROW;
      const int pcol = (((ov % R::VROW) / 16) ^ swz<8>(kr[i])) * 16;
      pbase[i] = vbase + kr[i] * vrs + pcol;
    }
  }
  // lane u < 2 loads tile u's bias (its position's row of log_prior)
  const int bpos = min(rpos[lane & 1], pend - 1);
  const float* bsrc = p.log_prior + ((int64_t)h * T + si.start + bpos) * g.C_slots;
  const int kmax = pend - 1;
  // loads of the block at key0 (chunk c for its bias) into a ring slot
  auto issue_at = [&](int key0, int c, uint32_t slot, uint32_t bslot) {
    if (!isk || key0 + 63 <= kmax) {
      const int64_t off = isk ? (int64_t)key0 * krs : (int64_t)key0 * 2;
#pragma unroll
      for (int i = 0; i < R::NP; ++i) lds_dma16(pbase[i] + off, slot + (wv * R::NP + i) * 1024);
    } else {
      // K rows past the sequence end (last chunk of the sequence): repeat the
      // last key instead of reading beyond it
#pragma unroll
      for (int i = 0; i < R::NP; ++i)
        lds_dma16(pbase[i] + (int64_t)(min(key0 + kr[i], kmax) - kr[i]) * krs,
                  slot + (wv * R::NP + i) * 1024);
    }
    // the tiles' biases for this block (past the routed blocks: any valid word)
    if (lane < 2) lds_dma4(bsrc + c, bslot + wv * 8);
  };
  // first key of step sx's block; c = its chunk for a routed block, else 0
  auto block_key0 = [&](int sx, int cl) -> int {
    return sx < nrouted ? cl * g.B + ((sx & sbl) << 6) : cdiag * g.B + ((sx - nrouted) << 6);
  };
  auto listed = [&](int sx) -> int {
    return sx < nrouted ? __builtin_amdgcn_readfirstlane((int)Blist[sx >> sbl]) : 0;
  };
  auto issue = [&](int sx, uint32_t slot, uint32_t bslot) {
    const int c = listed(sx);
    issue_at(block_key0(sx, c), c, slot, bslot);
  };

  // ---- tile state
  f32x4 o[2][DT];
  float l[2] = {0.f, 0.f};
  float m[2] = {-INFINITY, -INFINITY};
#pragma unroll
  for (int u = 0; u < 2; ++u)
#pragma unroll
    for (int dt = 0; dt < DT; ++dt) o[u][dt] = f32x4{0.f, 0.f, 0.f, 0.f};
  const float sl2 = p.scale * kLog2e;
  int koff[KS], voff[2];
#pragma unroll
  for (int ks = 0; ks < KS; ++ks) koff[ks] = r * R::KROW + (((4 * ks + gq) ^ swz<R::KP>(r)) * 16);
#pragma unroll
  for (int s2 = 0; s2 < 2; ++s2) voff[s2] = r * R::VROW + (((4 * s2 + gq) ^ swz<8>(r)) * 16);

  // Every step issues exactly one block's loads (past the end of the list it
  // re-reads the last block into the free slot, which no later step reads), so
  // when step st waits, exactly two blocks' loads are younger than its own:
  // one fixed counted wait proves slot st & 3 complete.
  const uint32_t ring0 = lds_addr(&ring[0][0]), bias0 = lds_addr(&bias[0][0]);
  __builtin_amdgcn_s_waitcnt(0 | (7 << 4));  // Q and mask reads done first
  issue(0, ring0, bias0);
  issue(min(1, NS - 1), ring0 + R::STAGE, bias0 + 4 * kRingTiles);
  issue(min(2, NS - 1), ring0 + 2 * R::STAGE, bias0 + 8 * kRingTiles);

  // wait for slot st & 3 and for every wave to be done with slot (st + 3) & 3;
  // returns the slot's LDS offset
  auto enter = [&](int st) -> lds_u8* {
    // own loads of this slot done (the two younger blocks may stay in flight),
    // this wave's LDS reads of the slot about to be refilled done
    __builtin_amdgcn_s_waitcnt(((2 * R::LPS) & 15) | (7 << 4));
    asm volatile("" ::: "memory");
    __builtin_amdgcn_s_barrier();
    asm volatile("" ::: "memory");
    return (lds_u8*)&ring[st & 3][0];
  };
  // refill of the slot released at the step's barrier (every wave was done
  // reading it) with the block three steps ahead
  auto leave = [&](int st, int cnext) {
    const int sr = st + 3, sx = min(sr, NS - 1);
    issue_at(block_key0(sx, cnext), cnext, ring0 + (sr & 3) * R::STAGE,
             bias0 + (sr & 3) * 4 * kRingTiles);
  };
  // routed blocks: each tile whose position has the chunk active visits it
  // with the tile's bias (the two visits, when both are active, run back to
  // back so that each tile's state is only ever updated in place)
  for (int st = 0; st < nrouted; ++st) {
    lds_u8* kv = enter(st);
    const int cnext = listed(min(st + 3, NS - 1));  // read now, used by the refill
    const uint32_t act = Act[st >> sbl];
    const bool a0 = rvalid[0] && ((act >> tpos[0]) & 1u);
    const bool a1 = rvalid[1] && ((act >> tpos[1]) & 1u);
    const float* bs = &bias[st & 3][2 * wv];
    const float bz[2] = {bs[0] * kLog2e, bs[1] * kLog2e};
    // a wave with nothing to visit issues the refill at once; a visiting wave
    // issues it afterwards, when the other waves' loads have left the queue
    if (!(a0 || a1)) leave(st, cnext);
    if (a0) visit_ring<D, false, 0, 1>(kv, kv + R::KBYTES, koff, voff, qa, o, l, m, sl2, bz, 0, rpos);
    if (a1) visit_ring<D, false, 1, 1>(kv, kv + R::KBYTES, koff, voff, qa, o, l, m, sl2, bz, 0, rpos);
    if (a0 || a1) leave(st, cnext);
  }
  // the diagonal chunk: both tiles, causal mask, bias 0, one fused visit
  for (int st = nrouted; st < NS; ++st) {
    lds_u8* kv = enter(st);
    const float bz[2] = {0.f, 0.f};
    const int key0 = cdiag * g.B + ((st - nrouted) << 6);
    if (rvalid[0])
      visit_ring<D, true, 0, 2>(kv, kv + R::KBYTES, koff, voff, qa, o, l, m, sl2, bz,
                                key0 + 4 * gq, rpos);
    leave(st, 0);
  }
  __builtin_amdgcn_s_waitcnt(0 | (7 << 4));  // no ring load outlives the kernel

#pragma unroll
  for (int u = 0; u < 2; ++u) {
    if (!rvalid[u]) continue;
    float lt = l[u] + xor16(l[u]);
    lt += xor32(lt);
    const float inv = 1.f / lt;
    const int64_t tok = si.start + rpos[u];
    uint16_t* orow = (uint16_t*)p.out + (tok * g.Hq + h * g.G + rhead[u]) * (int64_t)D;
#pragma unroll
    for (int dt = 0; dt < DT; ++dt) {
      const u32x2 w = {cvt_pk_bf16(o[u][dt][0] * inv, o[u][dt][1] * inv),
                       cvt_pk_bf16(o[u][dt][2] * inv, o[u][dt][3] * inv)};
      *reinterpret_cast<u32x2*>(orow + 16 * dt + 4 * gq) = w;
    }
    if (p.lse && gq == 0)
      p.lse[(int64_t)(h * g.G + rhead[u]) * T + tok] = (m[u] + __log2f(lt)) * kLn2;
  }
}

// ---------------------------------------------------------------- backward: dQ

// Backward of phase 2 for the queries, G >= 16, bf16 (the derivative of the
// prior-induced softmax attention: dS = P (dP - D), dQ = s dS K, and each
// routed chunk's bias gradient, the sum of dS over its keys and the group's
// heads).  The layout of work follows the forward ring kernel: 16 row tiles
// per workgroup (two per wave) walk the union of their positions' active
// blocks and the diagonal.  A block's K rows, V rows (both in the K layout)
// and K^T rows (from the transposed-K workspace, in the V^T layout) are staged
// in LDS, double-buffered, by plain vector loads.  Visit of an active tile:
// S^T = K Q^T and dP^T = V dO^T (16 MFMAs each), P^T = exp2(s S^T + b - LSE)
// from the forward's LSE, dS^T = P^T (dP^T - D) with D = <dO, O>, the tile's
// bias gradient sum(dS^T) added to dbias, and dQ^T += K^T dS^T (16 MFMAs).
// dQ (times s) is written in fp32 for the routing backward to add to.
// Blocks are staged by direct global->LDS loads (the swizzle applied on the
// source side), one block ahead, with a full vmcnt wait before each barrier.
constexpr int kBqWaves = 8;
constexpr int kBqThreads = 64 * kBqWaves;
constexpr int kBqTiles = 2 * kBqWaves;

template <int D>
__global__ __launch_bounds__(kBqThreads, 1) void bwd_dq_kernel(Geom g, BwdParams p, TileGeom tg) {
  constexpr int NTH = kBqThreads;
  using R = RingCfg<D>;
  constexpr int KS = D / 32;
  constexpr int DT = D / 16;
  constexpr int KB = R::KBYTES;           // K rows; V rows follow, then K^T rows
  constexpr int SB = 2 * KB + R::VBYTES;  // bytes of one staged block
  constexpr int NPC = SB / (16 * NTH);    // 16-byte pieces per thread
  static_assert(NPC * 16 * NTH == SB, "a block splits into whole pieces");
  __shared__ __attribute__((aligned(1024))) uint8_t stage[2][SB];
  __shared__ unsigned long long Umask[32];
  __shared__ int Wpref[33];
  __shared__ uint16_t Blist[2048];
  __shared__ uint16_t Act[2048];
  __shared__ float Bz[2][64];   // the staged block's bias per position (routed blocks)

  const int tid = threadIdx.x, lane = tid & 63;
  const int wv = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int r = lane & 15, gq = lane >> 4;
  const int tile = tg.tiles_per_seq - 1 - (int)blockIdx.x;
  const int s = blockIdx.y, h = blockIdx.z;
  const SeqInfo si = seq_info(g.cu_seqlens, nullptr, s, g.max_seqlen, g.B);
  const int p0 = tile * tg.P;
  if (p0 >= si.len) return;
  const int pend = min(p0 + tg.P, si.len);
  const int npos = pend - p0;
  const int cdiag = p0 / g.B;
  const int64_t T = g.T;
  const int W = g.W;
  const unsigned long long* __restrict__ mask = (const unsigned long long*)p.mask;

  int tpos[2], rpos[2], rhead[2];
  bool rvalid[2];
#pragma unroll
  for (int u = 0; u < 2; ++u) {
    const int ti = 2 * wv + u;
    tpos[u] = ti / tg.HT;
    rpos[u] = p0 + tpos[u];
    rhead[u] = (ti % tg.HT) * 16 + r;
    rvalid[u] = rpos[u] < pend;
  }
  // Q and dO operands (B of S^T = K Q^T and dP^T = V dO^T), the forward's LSE
  // and D = <dO, O> of the lane's head, in log2 units where they meet exp2
  bf16x8 qa[2][KS], da[2][KS];
  float lse2[2], dlt[2];
#pragma unroll
  for (int u = 0; u < 2; ++u) {
    const int64_t tok = si.start + min(rpos[u], pend - 1);
    const int64_t row = (tok * g.Hq + h * g.G + rhead[u]) * (int64_t)D;
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) {
      u32x4 a = {0u, 0u, 0u, 0u}, b = {0u, 0u, 0u, 0u};
      if (rvalid[u]) {
        a = ldg16((const uint16_t*)p.q + row + 32 * ks + 8 * gq);
        b = ldg16((const uint16_t*)p.dout + row + 32 * ks + 8 * gq);
      }
      qa[u][ks] = as_bf16x8(a);
      da[u][ks] = as_bf16x8(b);
    }
    const int64_t hr = (int64_t)(h * g.G + rhead[u]) * T + tok;
    lse2[u] = p.lse[hr] * kLog2e;
    dlt[u] = p.delta[hr];
  }

  // ---- the union of the positions' active chunks and their bitmap (as in
  // the forward kernel)
  if (tid < 32) Umask[tid] = 0ull;
  __syncthreads();
  const unsigned long long* mbase = mask + ((int64_t)h * T + si.start + p0) * W;
  for (int idx = tid; idx < npos * W; idx += NTH) {
    const int w = idx % W;
    const unsigned long long v = mbase[idx] & routable_bits(w, cdiag);
    if (v) atomicOr(&Umask[w], v);
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
    if (tid < 33) Wpref[tid] = inc - cnt;
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
  const int nlist = Wpref[W];
  for (int j = tid; j < nlist; j += NTH) {
    const int c = Blist[j];
    uint32_t bits = 0;
    for (int t = 0; t < npos; ++t)
      bits |= (uint32_t)((mbase[t * W + (c >> 6)] >> (c & 63)) & 1ull) << t;
    Act[j] = (uint16_t)bits;
  }
  __syncthreads();
  const int sbl = g.B == 128 ? 1 : 0;
  const int nrouted = nlist << sbl;
  const int ndiag = (pend - cdiag * g.B + 63) / 64;
  const int NS = nrouted + ndiag;

  // ---- staging: segment i of this wave is the 1 KB at (8 i + wv) KB of
  // the block; lane l fills its 16 bytes at l * 16, from the source piece that
  // the swizzled layout puts there (K and V rows in the K layout, K^T rows in
  // the V^T layout)
  const int kmax = pend - 1;  // last key of the sequence this workgroup may see
  const uint8_t* kb8 = (const uint8_t*)p.k + (si.start * (int64_t)g.Hkv + h) * D * 2;
  const uint8_t* vb8 = (const uint8_t*)p.v + (si.start * (int64_t)g.Hkv + h) * D * 2;
  const uint8_t* tb8 = (const uint8_t*)p.kt + (((int64_t)h * D) * p.Tp + pad_off(g, s)) * 2;
  auto block_key0 = [&](int sx) -> int {
    return sx < nrouted ? (int)Blist[sx >> sbl] * g.B + ((sx & sbl) << 6)
                        : cdiag * g.B + ((sx - nrouted) << 6);
  };
  const uint32_t krs = (uint32_t)(g.Hkv * D * 2);  // bytes between consecutive keys
  const uint32_t trs = (uint32_t)(p.Tp * 2);        // bytes between K^T rows
  auto sload = [&](int sx, int buf) {
    const int key0 = block_key0(sx);
    const uint32_t base = lds_addr(&stage[buf][0]);
#pragma unroll
    for (int i = 0; i < NPC; ++i) {
      const int seg = 8 * i + wv;  // wave-uniform: the segment lies in one region
      const int o = seg * 1024 + lane * 16;
      if (seg * 1024 < 2 * KB) {
        const int ok = o % KB;
        const int kr = ok / R::KROW;
        const int pc = ((ok % R::KROW) / 16) ^ swz<R::KP>(kr);
        const uint32_t key = (uint32_t)min(key0 + kr, kmax);
        lds_dma16s(seg * 1024 < KB ? kb8 : vb8, key * krs + (uint32_t)(pc * 16),
                   base + (uint32_t)(seg * 1024));
      } else {
        const int ot = o - 2 * KB;
        const int d = ot / R::VROW;
        const int pc = ((ot % R::VROW) / 16) ^ swz<8>(d);
        lds_dma16s(tb8, (uint32_t)d * trs + (uint32_t)(key0 * 2 + pc * 16),
                   base + (uint32_t)(seg * 1024));
      }
    }
    // a routed block's bias for each position, beside it (a load in the loop
    // itself would make the compiler wait for the whole staging)
    if (sx < nrouted && wv == 0 && lane < npos) {
      const int c = Blist[sx >> sbl];
      lds_dma4(p.log_prior + ((int64_t)h * T + si.start + p0 + lane) * g.C_slots + c,
               __builtin_amdgcn_readfirstlane(lds_addr(&Bz[buf][0])));
    }
  };

  f32x4 o[2][DT];
#pragma unroll
  for (int u = 0; u < 2; ++u)
#pragma unroll
    for (int dt = 0; dt < DT; ++dt) o[u][dt] = f32x4{0.f, 0.f, 0.f, 0.f};
  const float sl2 = p.scale * kLog2e;
  int koff[KS], voff[2];
#pragma unroll
  for (int ks = 0; ks < KS; ++ks) koff[ks] = r * R::KROW + (((4 * ks + gq) ^ swz<R::KP>(r)) * 16);
#pragma unroll
  for (int s2 = 0; s2 < 2; ++s2) voff[s2] = r * R::VROW + (((4 * s2 + gq) ^ swz<8>(r)) * 16);
  float* dbias = p.dbias;

  // one tile's visit of the staged block kv; returns the tile's sum of dS
  auto visit = [&](auto masked_tag, auto u_tag, lds_u8* kv, float bz, int kbase0) -> float {
    constexpr bool MASKED = decltype(masked_tag)::value;
    constexpr int U = decltype(u_tag)::value;
    f32x4 sacc[4], pacc[4];
#pragma unroll
    for (int t = 0; t < 4; ++t) {
      sacc[t] = f32x4{0.f, 0.f, 0.f, 0.f};
      pacc[t] = f32x4{0.f, 0.f, 0.f, 0.f};
    }
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) {
      u32x4 f[4];
#pragma unroll
      for (int t = 0; t < 4; ++t) f[t] = lds_read16(kv + koff[ks] + 16 * t * R::KROW);
#pragma unroll
      for (int t = 0; t < 4; ++t) sacc[t] = mfma16x16x32(as_bf16x8(f[t]), qa[U][ks], sacc[t]);
      __builtin_amdgcn_sched_barrier(0);
#pragma unroll
      for (int t = 0; t < 4; ++t) f[t] = lds_read16(kv + KB + koff[ks] + 16 * t * R::KROW);
#pragma unroll
      for (int t = 0; t < 4; ++t) pacc[t] = mfma16x16x32(as_bf16x8(f[t]), da[U][ks], pacc[t]);
      __builtin_amdgcn_sched_barrier(0);
    }
    uint32_t pk[4][2];
    float dsum = 0.f;
#pragma unroll
    for (int t = 0; t < 4; ++t) {
      float ds[4];
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        float pv = __builtin_amdgcn_exp2f(fmaf(sacc[t][j], sl2, bz - lse2[U]));
        if constexpr (MASKED) pv = kbase0 + 16 * t + j <= rpos[U] ? pv : 0.f;
        ds[j] = pv * (pacc[t][j] - dlt[U]);
        dsum += ds[j];
      }
      pk[t][0] = cvt_pk_bf16(ds[0], ds[1]);
      pk[t][1] = cvt_pk_bf16(ds[2], ds[3]);
    }
#pragma unroll
    for (int s2 = 0; s2 < 2; ++s2) {
      const u32x4 pb = {pk[2 * s2][0], pk[2 * s2][1], pk[2 * s2 + 1][0], pk[2 * s2 + 1][1]};
#pragma unroll
      for (int d0 = 0; d0 < DT; d0 += 4) {
        u32x4 a[4];
#pragma unroll
        for (int i = 0; i < 4; ++i)
          a[i] = lds_read16(kv + 2 * KB + voff[s2] + 16 * (d0 + i) * R::VROW);
#pragma unroll
        for (int i = 0; i < 4; ++i)
          o[U][d0 + i] = mfma16x16x32(as_bf16x8(a[i]), as_bf16x8(pb), o[U][d0 + i]);
        __builtin_amdgcn_sched_barrier(0);
      }
    }
    // the tile's sum of dS over its 16 heads and the block's keys
    dsum = row16_sum(dsum);
    dsum += xor16(dsum);
    dsum += xor32(dsum);
    return dsum;
  };
  using F = std::false_type;
  using Tr = std::true_type;
  using U0 = std::integral_constant<int, 0>;
  using U1 = std::integral_constant<int, 1>;

  __builtin_amdgcn_s_waitcnt(0 | (7 << 4));  // operand and mask reads done
  sload(0, 0);
  for (int st = 0; st < NS; ++st) {
    const int buf = st & 1;
    // this block's loads landed, every wave is done with the other buffer
    __builtin_amdgcn_s_waitcnt(0 | (7 << 4));
    asm volatile("" ::: "memory");
    __builtin_amdgcn_s_barrier();
    asm volatile("" ::: "memory");
    if (st + 1 < NS) sload(st + 1, buf ^ 1);
    lds_u8* kv = (lds_u8*)&stage[buf][0];
    if (st < nrouted) {
      const int c = Blist[st >> sbl];
      const uint32_t act = Act[st >> sbl];
#pragma unroll
      for (int u = 0; u < 2; ++u) {
        if (!(rvalid[u] && ((act >> tpos[u]) & 1u))) continue;
        const int64_t brow = ((int64_t)h * T + si.start + rpos[u]) * g.C_slots + c;
        const float bz = Bz[buf][tpos[u]] * kLog2e;
        const float d = u == 0 ? visit(F(), U0(), kv, bz, 0) : visit(F(), U1(), kv, bz, 0);
        if (lane == 0) atomicAdd(&dbias[brow], d);
      }
    } else {
      const int key0 = cdiag * g.B + ((st - nrouted) << 6);
      if (rvalid[0]) visit(Tr(), U0(), kv, 0.f, key0 + 4 * gq);
      if (rvalid[1]) visit(Tr(), U1(), kv, 0.f, key0 + 4 * gq);
    }
  }
  __builtin_amdgcn_s_waitcnt(0 | (7 << 4));  // no staging load outlives the kernel

  // dQ = s dQ^T^T, fp32: lane (gq, r) holds dims 16 dt + 4 gq .. +3 of head r
#pragma unroll
  for (int u = 0; u < 2; ++u) {
    if (!rvalid[u]) continue;
    const int64_t tok = si.start + rpos[u];
    float* drow = p.dq + (tok * g.Hq + h * g.G + rhead[u]) * (int64_t)D;
#pragma unroll
    for (int dt = 0; dt < DT; ++dt) {
      f32x4 w = o[u][dt];
#pragma unroll
      for (int j = 0; j < 4; ++j) w[j] *= p.scale;
      *reinterpret_cast<f32x4*>(drow + 16 * dt + 4 * gq) = w;
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

// Ring kernel (G >= 16): one 16-row tile per wave, 16 tiles, so P = 16 / (G / 16)
// positions per workgroup.
static TileGeom make_ring_tiles(const Geom& g) {
  TileGeom t;
  t.TP = 1;
  t.HT = g.G / 16;
  t.NT = kRingTiles;
  t.TW = 2;
  t.P = t.NT / t.HT;
  t.tiles_per_seq = (g.max_seqlen + t.P - 1) / t.P;
  return t;
}

bool prefill_uses_ring(const Geom& g) { return g.bf16 && g.G >= 16 && g.G <= 256; }

hipError_t launch_vt_transpose(const Geom& g, const void* src, void* dst, int64_t Tp,
                               hipStream_t st) {
  dim3 tgrid((g.max_seqlen + 63) / 64, g.num_seqs, g.Hkv);
  if (g.D == 64)
    hipLaunchKernelGGL(vt_transpose_kernel<64>, tgrid, dim3(256), 0, st, g,
                       (const uint16_t*)src, (uint16_t*)dst, Tp);
  else
    hipLaunchKernelGGL(vt_transpose_kernel<128>, tgrid, dim3(256), 0, st, g,
                       (const uint16_t*)src, (uint16_t*)dst, Tp);
  return hipGetLastError();
}

hipError_t launch_bwd_dq(const Geom& g, const BwdParams& p, hipStream_t st) {
  if (g.T == 0) return hipSuccess;
  const TileGeom rg = make_ring_tiles(g);
  dim3 grid(rg.tiles_per_seq, g.num_seqs, g.Hkv);
  if (g.D == 64)
    hipLaunchKernelGGL(bwd_dq_kernel<64>, grid, dim3(kBqThreads), 0, st, g, p, rg);
  else
    hipLaunchKernelGGL(bwd_dq_kernel<128>, grid, dim3(kBqThreads), 0, st, g, p, rg);
  return hipGetLastError();
}

hipError_t launch_prefill_attn(const Geom& g, const PrefillParams& p, hipStream_t st) {
  if (g.T == 0) return hipSuccess;
  if (g.bf16) {
    const TileGeom tg = make_tiles(g);
    dim3 grid(tg.tiles_per_seq, g.num_seqs, g.Hkv);
    if (prefill_uses_ring(g)) {
      const TileGeom rg = make_ring_tiles(g);
      dim3 rgrid(rg.tiles_per_seq, g.num_seqs, g.Hkv);
      dim3 tgrid((g.max_seqlen + 63) / 64, g.num_seqs, g.Hkv);
      if (g.D == 64) {
        hipLaunchKernelGGL(vt_transpose_kernel<64>, tgrid, dim3(256), 0, st, g,
                           (const uint16_t*)p.v, (uint16_t*)p.vt, p.Tp);
        hipLaunchKernelGGL(prefill_attn_ring_kernel<64>, rgrid, dim3(kRingThreads), 0, st, g,
                           p, rg);
      } else {
        hipLaunchKernelGGL(vt_transpose_kernel<128>, tgrid, dim3(256), 0, st, g,
                           (const uint16_t*)p.v, (uint16_t*)p.vt, p.Tp);
        hipLaunchKernelGGL(prefill_attn_ring_kernel<128>, rgrid, dim3(kRingThreads), 0, st, g,
                           p, rg);
      }
      return hipGetLastError();
    }
#define DASH_PRE(DD, U)                                                                   \
  hipLaunchKernelGGL((prefill_attn_bf16_kernel<DD, U>), grid, dim3(kPrefillThreads), 0, st, \
                     g, p, tg)
    if (g.D == 64) DASH_PRE(64, false); else DASH_PRE(128, false);
#undef DASH_PRE
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
