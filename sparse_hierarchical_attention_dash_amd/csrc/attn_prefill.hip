// Phase 2, prefill: prior-induced sparse softmax attention ("Fase 2:
// Prior-Geinduceerde Spaarzame Softmax" of the gist.science technical summary:
// a FlashAttention-style loop over the active chunks of a bit-packed mask,
// the routing bias added to the logits before the softmax, and a separate
// diagonal branch for the query's own chunk).
//
// Three kernels:
//   * prefill_attn_ring_kernel (bf16, GQA group G >= 16): a 16-row MFMA tile
//     is the 16 query heads of one position, so tiles share their mask.  A
//     workgroup owns 16 tiles (16 waves of one tile for groups of 16 heads, 8
//     waves of one position's two tiles for groups of 32) and streams the
//     union of its positions' active chunks, then its diagonal blocks, through a
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

// LDS layout of one staged 64-key block: K rows, then V^T rows.
template <int D>
struct RingCfg {
  static constexpr int KROW = D * 2;                  // bytes per K row
  static constexpr int KP = KROW / 16;                // 16-byte pieces per K row
  static constexpr int KBYTES = 64 * KROW;
  static constexpr int VROW = 128;                    // bytes per V^T row (64 keys)
  static constexpr int VBYTES = D * VROW;
  static constexpr int STAGE = KBYTES + VBYTES;
};
// How NTH threads split a block's staging: NP 16-byte loads each, a wave's
// pieces lying all in K or all in V^T.
template <int D, int NTH>
struct RingSplit {
  using R = RingCfg<D>;
  static constexpr int NP = R::STAGE / (16 * NTH);  // 16-byte loads per thread
  static constexpr int LPS = NP + 1;                 // + the tiles' bias words
  static_assert(NP * 16 * NTH == R::STAGE, "slot must split into whole loads");
  static_assert(R::KBYTES % (NP * 1024) == 0, "a wave's pieces lie all in K or all in V^T");
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
template <int D, bool MASKED, int U0, int NTL, int TWN = 2, int NFR = 3>
__device__ __forceinline__ void visit_ring(lds_u8* ks_, lds_u8* vt_,
                                           const int (&koff)[D / 32], const int (&voff)[2],
                                           const bf16x8 (&qa)[TWN][D / 32],
                                           f32x4 (&o)[TWN][D / 16], float (&l)[TWN],
                                           float (&m)[TWN], float sl2, const float (&bz)[TWN],
                                           int kbase, const int (&rpos)[TWN]) {
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
  // fragment groups 0 .. KS-1 are K (ks = g), KS .. KS+NVG-1 are V^T; NFR
  // buffers, NFR - 1 groups in flight ahead of the one being consumed
  constexpr int NG = KS + NVG;
  constexpr int AH = NFR - 1;
  u32x4 fr[NFR][4];
  auto gload = [&](int gi) {
    if (gi < KS) kload(fr[gi % NFR], gi);
    else if (gi < NG) vload(fr[gi % NFR], gi - KS);
  };
  f32x4 sacc[NTL][4];
#pragma unroll
  for (int u = 0; u < NTL; ++u)
#pragma unroll
    for (int t = 0; t < 4; ++t) sacc[u][t] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
  for (int a = 0; a < AH; ++a) gload(a);
#pragma unroll
  for (int ks = 0; ks < KS; ++ks) {
    gload(ks + AH);
    __builtin_amdgcn_sched_barrier(0);
#pragma unroll
    for (int t = 0; t < 4; ++t)
#pragma unroll
      for (int u = 0; u < NTL; ++u)
        sacc[u][t] = mfma16x16x32(as_bf16x8(fr[ks % NFR][t]), qa[U0 + u][ks], sacc[u][t]);
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
    gload(KS + vg + AH);
    __builtin_amdgcn_sched_barrier(0);
    const int s2 = vg / (DT / 4), dt0 = 4 * (vg % (DT / 4));
    u32x4 (&cur)[4] = fr[(KS + vg) % NFR];
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

// The ordered list of the union of a workgroup's positions' active chunks
// (Blist), for each listed chunk the positions that have it active (Act, bit
// t: the workgroup's position t), and with 64-key chunks the visiting order
// (the list permuted in place); returns the list's length.  mbase: the mask
// row of the workgroup's first position (W words a row), npos positions,
// cdiag the positions' own chunk (not routable); HT tiles per position.
// Every thread of the workgroup calls it.
template <int NWV, int TW, typename ActT>
__device__ __forceinline__ int ring_build_list(int W, int HT, bool b128,
                                               const unsigned long long* __restrict__ mbase,
                                               int npos, int cdiag, unsigned long long* Umask,
                                               int* Wpref, uint16_t* Blist, ActT* Act,
                                               uint16_t* Ord) {
  constexpr int NTH = 64 * NWV;
  const int tid = threadIdx.x, lane = tid & 63;
  const int wv = __builtin_amdgcn_readfirstlane(tid >> 6);
  if (tid < 32) Umask[tid] = 0ull;
  __syncthreads();
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
    Act[j] = (ActT)bits;
  }
  __syncthreads();

  // visiting order (64-key chunks).  The loop below takes two listed
  // chunks per barrier, so the wait at a barrier is for the busiest wave over
  // both; they are paired so that their active tiles fall on different
  // waves.  Wave w pairs the entries of list blocks w, w + NWV, ... (64
  // entries each) greedily: the first unpaired entry i of the block takes
  // the first unpaired entry after it that keeps the pair's load lowest.
  // With two tiles a wave: every wave at one visit, else at two, else any
  // (v packs per wave, 4 bits each, the tile visits of an entry; a sum of two
  // never carries between the fields).  With one tile a wave: the busiest
  // SIMD's visits, then whether some wave visits twice (16 waves x 1 tile:
  // 64K attention 15.1 -> 14.9 ms against the wave rule alone).
  if (!b128 && nlist > 2) {
    for (int b = wv; b * 64 < nlist; b += NWV) {
      const int e = b * 64 + lane;
      uint32_t v = 0;
      if (e < nlist) {
        const uint32_t act = Act[e];
        if constexpr (TW == 1) {
          // one tile a wave: a bit per wave
#pragma unroll
          for (int w = 0; w < NWV; ++w) v |= ((act >> (w / HT)) & 1u) << w;
        } else {
#pragma unroll
          for (int w = 0; w < NWV; ++w) {
            uint32_t c = 0;
#pragma unroll
            for (int u = 0; u < TW; ++u) c += (act >> ((TW * w + u) / HT)) & 1u;
            v |= c << (4 * w);
          }
        }
      }
      uint64_t taken = ~__ballot(e < nlist);
      // one tile a wave: the visits per SIMD too (4 bits each), taking wave w
      // to run on SIMD w % 4 (waves are placed on the four SIMDs in turn)
      uint32_t sl = 0;
      if constexpr (TW == 1) {
#pragma unroll
        for (int q = 0; q < 4; ++q) sl |= (uint32_t)__popc(v & (0x1111u << q)) << (4 * q);
      }
      int out = b * 64;
      while (~taken) {
        const int i = __ffsll((long long)~taken) - 1;
        taken |= 1ull << i;
        const uint32_t vi = (uint32_t)__builtin_amdgcn_readlane((int)v, i);
        const uint32_t t = vi + v;
        int j = -1;
        if constexpr (TW == 1) {
          // the partner keeping the busiest SIMD lowest, then no wave twice
          const uint32_t ts = (uint32_t)__builtin_amdgcn_readlane((int)sl, i) + sl;
          const uint32_t mx = max(max(ts & 15u, (ts >> 4) & 15u), max((ts >> 8) & 15u, ts >> 12));
          int k = ((taken >> lane) & 1ull) ? 64 : (int)(2 * mx + ((vi & v) ? 1u : 0u));
          int km = k;
#pragma unroll
          for (int o = 1; o < 64; o <<= 1) km = min(km, __shfl_xor(km, o));
          if (km < 64) j = __ffsll((long long)__ballot(k == km)) - 1;
        } else {
        // 1: no wave visits twice, 2: at most twice, 3: more; 4: taken
        const bool ge2 = TW == 1 ? (vi & v) != 0u : ((t + 0x66666666u) & 0x88888888u) != 0u;
        const bool ge3 = TW == 1 ? false : ((t + 0x55555555u) & 0x88888888u) != 0u;
        const int k = ((taken >> lane) & 1ull) ? 4 : (ge3 ? 3 : (ge2 ? 2 : 1));
        for (int cls = 1; cls <= 3 && j < 0; ++cls) {
          const uint64_t bm = __ballot(k <= cls);
          if (bm) j = __ffsll((long long)bm) - 1;
        }
        }
        if (lane == 0) {
          Ord[out] = (uint16_t)(b * 64 + i);
          if (j >= 0) Ord[out + 1] = (uint16_t)(b * 64 + j);
        }
        out += j >= 0 ? 2 : 1;
        if (j >= 0) taken |= 1ull << j;
      }
    }
    __syncthreads();
    constexpr int PER = (2048 + NTH - 1) / NTH;
    uint16_t tb[PER];
    ActT ta[PER];
#pragma unroll
    for (int q = 0; q < PER; ++q) {
      const int j = tid + q * NTH;
      if (j < nlist) {
        const int o = Ord[j];
        tb[q] = Blist[o];
        ta[q] = Act[o];
      }
    }
    __syncthreads();
#pragma unroll
    for (int q = 0; q < PER; ++q) {
      const int j = tid + q * NTH;
      if (j < nlist) {
        Blist[j] = tb[q];
        Act[j] = ta[q];
      }
    }
    __syncthreads();
  }
  return nlist;
}

// Prefill attention for G >= 16 (every 16-row tile is 16 query heads of one
// position).  A workgroup of NWV waves owns NT = NWV * TW tiles, TW per wave,
// so P = NT / (G / 16) positions (P divides B: the positions share one
// diagonal chunk).  The blocks of the workgroup's list stream through a
// 4-slot LDS ring filled by direct global->LDS loads (K rows from K, V^T rows
// from the V^T workspace, and each tile's bias for the block): with 64-key
// chunks two blocks per barrier, the next two loading meanwhile; with
// 128-key chunks one block per barrier, three blocks ahead.  Which positions
// have each listed chunk active is worked out once, up front, into a bitmap
// in LDS, so the loop reads no memory but LDS.  Waits are counted (vmcnt) and
// the barrier carries no fence.
//   PAIR: a wave's tiles 2k and 2k+1 always share their position (G = 32), so
//         they visit together and every LDS fragment feeds both; otherwise
//         each active tile visits alone.
//   NFR : LDS fragment groups in flight per visit (register budget).
// Work items: `items` (varlen packs) lists (sequence << 16 | tile) in the
// cost-sorted order of prefill_schedule_kernel, 0xffffffff past its end;
// without it a fixed-length batch maps item w to tile tiles_per_seq - 1 -
// w % tiles_per_seq of sequence w / tiles_per_seq (each sequence's tiles
// costliest first).  blockIdx.x = item, blockIdx.y = KV head (one head's
// keys and values at a time in the caches).
template <int D, int NWV, int TW, bool PAIR, int NFR>
__global__ __launch_bounds__(64 * NWV, 1) void prefill_attn_ring_kernel(
    Geom g, PrefillParams p, TileGeom tg, const uint32_t* __restrict__ items) {
  constexpr int NTH = 64 * NWV;
  constexpr int NT = NWV * TW;
  using R = RingCfg<D>;
  using RS = RingSplit<D, NTH>;
  constexpr int NP = RS::NP;
  constexpr int KS = D / 32;
  constexpr int DT = D / 16;
  static_assert(NT <= 32, "one activity word per listed chunk");
  static_assert(!PAIR || TW % 2 == 0, "pairs of tiles");
  static_assert(TW == 1 ? NWV <= 32 : NWV <= 8, "per-wave visit counts packed in 32 bits");
  __shared__ __attribute__((aligned(1024))) uint8_t ring[kRing][R::STAGE];
  __shared__ float bias[kRing][NT];
  __shared__ unsigned long long Umask[32];
  __shared__ int Wpref[33];
  __shared__ uint16_t Blist[2048];
  using ActT = typename std::conditional<NT <= 16, uint16_t, uint32_t>::type;
  __shared__ ActT Act[2048];   // bit t: position p0 + t has chunk Blist[j] active
  __shared__ uint16_t Ord[2048];  // visiting order of the list (64-key chunks)

  const int tid = threadIdx.x, lane = tid & 63;
  const int wv = __builtin_amdgcn_readfirstlane(tid >> 6);  // wave index, held in an SGPR
  const int r = lane & 15, gq = lane >> 4;
  const int h = blockIdx.y;
  const int w_item = blockIdx.x;
  int s, tile;
  if (items) {
    const uint32_t it = items[w_item];
    if (it == 0xffffffffu) return;
    s = (int)(it >> 16);
    tile = (int)(it & 0xffffu);
  } else {
    s = w_item / tg.tiles_per_seq;
    tile = tg.tiles_per_seq - 1 - w_item % tg.tiles_per_seq;
  }
  const SeqInfo si = seq_info(g.cu_seqlens, nullptr, s, g.max_seqlen, g.B);
  const int p0 = tile * tg.P;
  if (p0 >= si.len) return;
  const int pend = min(p0 + tg.P, si.len);
  const int npos = pend - p0;
  const int cdiag = p0 / g.B;
  const int64_t T = g.T;
  const int W = g.W;
  const unsigned long long* __restrict__ mask = (const unsigned long long*)p.mask;

  // this wave's tiles u < TW: 16 heads (rhead) of position rpos = p0 + tpos
  int tpos[TW], rpos[TW], rhead[TW];
  bool rvalid[TW];
#pragma unroll
  for (int u = 0; u < TW; ++u) {
    const int ti = TW * wv + u;
    tpos[u] = ti / tg.HT;
    rpos[u] = p0 + tpos[u];
    rhead[u] = (ti % tg.HT) * 16 + r;
    rvalid[u] = rpos[u] < pend;
  }
  bf16x8 qa[TW][KS];
#pragma unroll
  for (int u = 0; u < TW; ++u) {
    const int64_t qrow = ((si.start + rpos[u]) * g.Hq + h * g.G + rhead[u]) * (int64_t)D;
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) {
      u32x4 v = {0u, 0u, 0u, 0u};
      if (rvalid[u]) v = ldg16((const uint16_t*)p.q + qrow + 32 * ks + 8 * gq);
      qa[u][ks] = as_bf16x8(v);
    }
  }

  // ---- ordered list of the union of the positions' active chunks, the
  // positions that have each listed chunk active, and the visiting order
  const unsigned long long* mbase = mask + ((int64_t)h * T + si.start + p0) * W;
  const int nlist = ring_build_list<NWV, TW>(W, tg.HT, g.B == 128, mbase, npos, cdiag, Umask,
                                             Wpref, Blist, Act, Ord);
  const int sbl = g.B == 128 ? 1 : 0;  // log2 of the 64-key blocks per chunk
  const int nrouted = nlist << sbl;
  const int ndiag = (pend - cdiag * g.B + 63) / 64;
  const int NS = nrouted + ndiag;

  // ---- per-thread DMA sources (piece layout fixed per thread; a wave's
  // pieces are all K rows or all V^T rows)
  const int64_t krs = (int64_t)g.Hkv * D * 2;  // bytes between consecutive keys
  const int64_t vrs = p.Tp * 2;                  // bytes between V^T rows
  const bool isk = wv * NP * 1024 < R::KBYTES;
  const uint8_t* kbase = (const uint8_t*)p.k + (si.start * (int64_t)g.Hkv + h) * D * 2;
  const uint8_t* vbase = (const uint8_t*)p.vt + ((int64_t)h * D * p.Tp + pad_off(g, s)) * 2;
  // piece i of this thread: K row or V^T row kr(i) of the block, at source
  // address pbase[i] + (K: key0 * krs, V^T: key0 * 2) for the block at key0
  auto krow = [&](int i) -> int {
    const int o = (wv * NP + i) * 1024 + lane * 16;
    return isk ? o / R::KROW : (o - R::KBYTES) / R::VROW;
  };
  const uint8_t* pbase[NP];
#pragma unroll
  for (int i = 0; i < NP; ++i) {
    const int o = (wv * NP + i) * 1024 + lane * 16;
    const int kr = krow(i);
    if (isk) {
      const int pcol = (((o % R::KROW) / 16) ^ swz<R::KP>(kr)) * 16;
      pbase[i] = kbase + kr * krs + pcol;
    } else {
      const int pcol = ((((o - R::KBYTES) % R::VROW) / 16) ^ swz<8>(kr)) * 16;
      pbase[i] = vbase + kr * vrs + pcol;
    }
  }
  // lane u < TW loads tile (TW * wv + u)'s bias (its position's row of log_prior)
  const int bpos = min(p0 + (TW * wv + min(lane, TW - 1)) / tg.HT, pend - 1);
  const float* bsrc = p.log_prior + ((int64_t)h * T + si.start + bpos) * g.C_slots;
  const int kmax = pend - 1;
  // loads of the block at key0 (chunk c for its bias) into a ring slot
  auto issue_at = [&](int key0, int c, uint32_t slot, uint32_t bslot) {
    if (!isk || key0 + 63 <= kmax) {
      const int64_t off = isk ? (int64_t)key0 * krs : (int64_t)key0 * 2;
#pragma unroll
      for (int i = 0; i < NP; ++i) lds_dma16(pbase[i] + off, slot + (wv * NP + i) * 1024);
    } else {
      // K rows past the sequence end (last chunk of the sequence): repeat the
      // last key instead of reading beyond it
#pragma unroll
      for (int i = 0; i < NP; ++i) {
        const int kr = krow(i);
        lds_dma16(pbase[i] + (int64_t)(min(key0 + kr, kmax) - kr) * krs,
                  slot + (wv * NP + i) * 1024);
      }
    }
    // the tiles' biases for this block (past the routed blocks: any valid word)
    if (lane < TW) lds_dma4(bsrc + c, bslot + wv * TW * 4);
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
  f32x4 o[TW][DT];
  float l[TW], m[TW];
#pragma unroll
  for (int u = 0; u < TW; ++u) {
    l[u] = 0.f;
    m[u] = -INFINITY;
#pragma unroll
    for (int dt = 0; dt < DT; ++dt) o[u][dt] = f32x4{0.f, 0.f, 0.f, 0.f};
  }
  const float sl2 = p.scale * kLog2e;
  int koff[KS], voff[2];
#pragma unroll
  for (int ks = 0; ks < KS; ++ks) koff[ks] = r * R::KROW + (((4 * ks + gq) ^ swz<R::KP>(r)) * 16);
#pragma unroll
  for (int s2 = 0; s2 < 2; ++s2) voff[s2] = r * R::VROW + (((4 * s2 + gq) ^ swz<8>(r)) * 16);

  const uint32_t ring0 = lds_addr(&ring[0][0]), bias0 = lds_addr(&bias[0][0]);
  // the wave's tiles whose position has listed chunk j active (bit u: tile u)
  auto active_mask = [&](int j) -> uint32_t {
    const uint32_t act = Act[j];
    uint32_t am = 0;
#pragma unroll
    for (int u = 0; u < TW; ++u)
      am |= (rvalid[u] && ((act >> tpos[u]) & 1u)) ? (1u << u) : 0u;
    return am;
  };
  // routed block of step st in slot kv: the active tiles visit it with their
  // biases; tiles of one position (PAIR) visit together, every LDS fragment
  // feeding both.  (Two tiles of different positions visiting together when
  // both are active measured slower than one after the other: the fused visit
  // fits the register budget only without fragment prefetch.)
  auto routed_step = [&](int st, lds_u8* kv, uint32_t am) {
    float bz[TW];
    const float* bs = &bias[st & 3][TW * wv];
#pragma unroll
    for (int u = 0; u < TW; ++u) bz[u] = bs[u] * kLog2e;
    static_for<0, (PAIR ? TW / 2 : TW)>([&](auto k_) {
      constexpr int U0 = PAIR ? 2 * decltype(k_)::value : decltype(k_)::value;
      if ((am >> U0) & 1u)
        visit_ring<D, false, U0, PAIR ? 2 : 1, TW, NFR>(kv, kv + R::KBYTES, koff, voff, qa, o, l,
                                                         m, sl2, bz, 0, rpos);
    });
  };
  // diagonal block of step st: every tile, causal mask, bias 0 (two at a time)
  auto diag_step = [&](int st, lds_u8* kv) {
    float bz[TW];
#pragma unroll
    for (int u = 0; u < TW; ++u) bz[u] = 0.f;
    const int key0 = cdiag * g.B + ((st - nrouted) << 6);
    if constexpr (TW == 1) {
      if (rvalid[0])
        visit_ring<D, true, 0, 1, TW, NFR>(kv, kv + R::KBYTES, koff, voff, qa, o, l, m, sl2, bz,
                                           key0 + 4 * gq, rpos);
    } else {
      static_for<0, TW / 2>([&](auto k_) {
        constexpr int U0 = 2 * decltype(k_)::value;
        if (rvalid[U0])
          visit_ring<D, true, U0, 2, TW, NFR>(kv, kv + R::KBYTES, koff, voff, qa, o, l, m, sl2,
                                              bz, key0 + 4 * gq, rpos);
      });
    }
  };
  __builtin_amdgcn_s_waitcnt(0 | (7 << 4));  // Q and mask reads done first
  if (sbl == 0) {
    // Chunks of 64 keys: two blocks per barrier.  Step st (even) waits for
    // its own loads of blocks st and st + 1, and at its barrier every wave has
    // left blocks st - 2 and st - 1, whose slots then take blocks st + 2 and
    // st + 3.  A wave then visits its tiles of both blocks before the next
    // barrier, so the wait at a barrier is for the busiest wave over two
    // blocks rather than over each one (the active tiles of two different
    // chunks even out between the waves; 64K prefill 18.4 -> 16.5 ms).
    issue(0, ring0, bias0);
    if (NS > 1) issue(1, ring0 + R::STAGE, bias0 + 4 * NT);
    auto pair_enter = [&](int st) {
      if (st & 1) return;
      wait_vm<0>();
      asm volatile("" ::: "memory");
      __builtin_amdgcn_s_barrier();
      asm volatile("" ::: "memory");
#pragma unroll 1
      for (int b = st + 2; b < min(st + 4, NS); ++b)
        issue(b, ring0 + (b & 3) * R::STAGE, bias0 + (b & 3) * 4 * NT);
    };
    // (one visit per iteration: a loop over the pair's two blocks made the
    // compiler move every O accumulator between registers each step)
    for (int st = 0; st < nrouted; ++st) {
      pair_enter(st);
      routed_step(st, (lds_u8*)&ring[st & 3][0], active_mask(st));
    }
    for (int st = nrouted; st < NS; ++st) {
      pair_enter(st);
      diag_step(st, (lds_u8*)&ring[st & 3][0]);
    }
  } else {
    // Chunks of 128 keys: both blocks of a chunk have the same active tiles,
    // so pairing them evens nothing out; one block per barrier, loads three
    // blocks ahead.  Every step issues exactly one block's loads (past the end
    // of the list it re-reads the last block into the free slot, which no
    // later step reads), so when step st waits, exactly two blocks' loads are
    // younger than its own: one fixed counted wait proves slot st & 3
    // complete.
    issue(0, ring0, bias0);
    issue(min(1, NS - 1), ring0 + R::STAGE, bias0 + 4 * NT);
    issue(min(2, NS - 1), ring0 + 2 * R::STAGE, bias0 + 8 * NT);
    // wait for slot st & 3 and for every wave to be done with slot (st + 3) & 3
    auto enter = [&](int st) -> lds_u8* {
      // own loads of this slot done (the two younger blocks may stay in
      // flight), this wave's LDS reads of the slot about to be refilled done
      wait_vm<2 * RS::LPS>();
      asm volatile("" ::: "memory");
      __builtin_amdgcn_s_barrier();
      asm volatile("" ::: "memory");
      return (lds_u8*)&ring[st & 3][0];
    };
    // refill of the slot released at the step's barrier with the block three
    // steps ahead
    auto leave = [&](int st, int cnext) {
      const int sr = st + 3, sx = min(sr, NS - 1);
      issue_at(block_key0(sx, cnext), cnext, ring0 + (sr & 3) * R::STAGE,
               bias0 + (sr & 3) * 4 * NT);
    };
    for (int st = 0; st < nrouted; ++st) {
      lds_u8* kv = enter(st);
      const int cnext = listed(min(st + 3, NS - 1));  // read now, used by the refill
      const uint32_t am = active_mask(st >> sbl);
      // a wave with nothing to visit issues the refill at once; a visiting
      // wave issues it afterwards, when the other waves' loads have left the
      // queue
      if (!am) leave(st, cnext);
      routed_step(st, kv, am);
      if (am) leave(st, cnext);
    }
    for (int st = nrouted; st < NS; ++st) {
      lds_u8* kv = enter(st);
      diag_step(st, kv);
      leave(st, 0);
    }
  }
  __builtin_amdgcn_s_waitcnt(0 | (7 << 4));  // no ring load outlives the kernel

#pragma unroll
  for (int u = 0; u < TW; ++u) {
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
// heads).  The work is laid out as in the forward ring kernel: 16 row tiles
// per workgroup (one a wave for G = 16, a pair of one position for G = 32)
// walk the union of their positions' active blocks (ring_build_list, paired
// for 64-key chunks) and then the diagonal, through the same 4-slot LDS ring
// and barrier schedule.  A staged block is the block's K rows and V rows,
// 16-byte pieces XOR-swizzled by head_row_swz; K^T, the operand of the dQ product,
// comes from the K rows by gfx950's transposing LDS reads, so a block crosses
// the fabric once, as 2 x 64 rows.  Visit of an active tile, 32 keys at a
// time: S^T = K Q^T and dP^T = V dO^T (16x16x32), P^T = exp2(s S^T + b - LSE)
// from the forward's LSE, dS^T = P^T (dP^T - D) with D = <dO, O>, dQ^T +=
// K^T dS^T (16x16x32); a routed block's bias gradient, the tile's sum of dS,
// is added atomically.  dQ (times s) is written in fp32 for the routing
// backward to add to.

// One visit of tiles U0 .. U0+NTL-1 of a wave to one staged block (K rows at
// ks_, V rows at vs_), in two halves of 32 keys.  koff: the lane's S^T / dP^T
// operand offsets (row r, piece 4 ks + gq); tb, tx: the transposing reads'
// row offset and swizzle (below).  Adds each tile's partial sum of dS to
// dsum.  MASKED: key j of the block is seen iff kbase + j - 4 gq <= the
// tile's position (kbase = the block's first key + 4 gq).
template <int D, bool MASKED, int U0, int NTL, int TWN>
__device__ __forceinline__ void visit_dq(lds_u8* ks_, lds_u8* vs_, const int (&koff)[D / 32],
                                         int tb, int tx, const bf16x8 (&qa)[TWN][D / 32],
                                         const bf16x8 (&da)[TWN][D / 32],
                                         const float (&lse2)[TWN], const float (&dlt)[TWN],
                                         f32x4 (&o)[TWN][D / 16], float (&dsum)[TWN], float sl2,
                                         const float (&bz)[TWN], int kbase,
                                         const int (&rpos)[TWN]) {
  constexpr int KROW = 2 * D;
  constexpr int KS = D / 32;
  constexpr int DT = D / 16;
#pragma unroll
  for (int h2 = 0; h2 < 2; ++h2) {
    // S^T and dP^T of keys 32 h2 .. +31 (key tiles t = 0, 1 of the half):
    // lane (gq, r) holds keys 32 h2 + 16 t + 4 gq + j of head r
    f32x4 sacc[NTL][2], pacc[NTL][2];
#pragma unroll
    for (int u = 0; u < NTL; ++u)
#pragma unroll
      for (int t = 0; t < 2; ++t) {
        sacc[u][t] = f32x4{0.f, 0.f, 0.f, 0.f};
        pacc[u][t] = f32x4{0.f, 0.f, 0.f, 0.f};
      }
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) {
      u32x4 fk[2], fv[2];
#pragma unroll
      for (int t = 0; t < 2; ++t) {
        fk[t] = lds_read16(ks_ + koff[ks] + (32 * h2 + 16 * t) * KROW);
        fv[t] = lds_read16(vs_ + koff[ks] + (32 * h2 + 16 * t) * KROW);
      }
#pragma unroll
      for (int t = 0; t < 2; ++t)
#pragma unroll
        for (int u = 0; u < NTL; ++u) {
          sacc[u][t] = mfma16x16x32(as_bf16x8(fk[t]), qa[U0 + u][ks], sacc[u][t]);
          pacc[u][t] = mfma16x16x32(as_bf16x8(fv[t]), da[U0 + u][ks], pacc[u][t]);
        }
    }
    // dS^T, packed as the B operand of dQ^T += K^T dS^T: k-slot 8 gq + 4 t + j
    // is key 32 h2 + 16 t + 4 gq + j
    u32x4 pb[NTL];
#pragma unroll
    for (int u = 0; u < NTL; ++u) {
      const float off = bz[U0 + u] - lse2[U0 + u];
      float ds[2][4];
#pragma unroll
      for (int t = 0; t < 2; ++t)
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          float pv = __builtin_amdgcn_exp2f(fmaf(sacc[u][t][j], sl2, off));
          if constexpr (MASKED) pv = kbase + 32 * h2 + 16 * t + j <= rpos[U0 + u] ? pv : 0.f;
          ds[t][j] = pv * (pacc[u][t][j] - dlt[U0 + u]);
          dsum[U0 + u] += ds[t][j];
        }
      pb[u] = u32x4{cvt_pk_bf16(ds[0][0], ds[0][1]), cvt_pk_bf16(ds[0][2], ds[0][3]),
                    cvt_pk_bf16(ds[1][0], ds[1][1]), cvt_pk_bf16(ds[1][2], ds[1][3])};
    }
    // K^T operand of dims 16 dt .. +15: two transposing reads, of key rows
    // 32 h2 + 4 gq + r / 4 and the same + 16, give lane (gq, r) dim 16 dt + r
    // of the keys of its k-slots
#pragma unroll
    for (int dt = 0; dt < DT; ++dt) {
      lds_u8* a = ks_ + tb + 32 * h2 * KROW + 32 * (dt ^ tx);
      const s16x4 a0 = lds_read_tr8(a), a1 = lds_read_tr8(a + 16 * KROW);
      const bf16x8 ka = __builtin_bit_cast(
          bf16x8, u32x4{__builtin_bit_cast(u32x2, a0)[0], __builtin_bit_cast(u32x2, a0)[1],
                        __builtin_bit_cast(u32x2, a1)[0], __builtin_bit_cast(u32x2, a1)[1]});
#pragma unroll
      for (int u = 0; u < NTL; ++u)
        o[U0 + u][dt] = mfma16x16x32(ka, as_bf16x8(pb[u]), o[U0 + u][dt]);
    }
  }
}

template <int D, int NWV, int TW, bool PAIR>
__global__ __launch_bounds__(64 * NWV, 1) void bwd_dq_ring_kernel(Geom g, BwdParams p,
                                                                  TileGeom tg) {
  constexpr int NTH = 64 * NWV;
  constexpr int NT = NWV * TW;
  constexpr int KROW = 2 * D;
  constexpr int KBYTES = 64 * KROW;
  constexpr int STAGE = 2 * KBYTES;       // K rows, then V rows
  constexpr int NP = STAGE / (16 * NTH);  // 16-byte loads per thread per block
  constexpr int LPS = NP + 1;             // + the tiles' bias words
  constexpr int KS = D / 32;
  constexpr int DT = D / 16;
  static_assert(NP * 16 * NTH == STAGE, "a block splits into whole loads");
  static_assert(KBYTES % (NP * 1024) == 0, "a wave's pieces lie all in K or all in V");
  static_assert(NT <= 16, "one 16-bit activity word per listed chunk");
  static_assert(!PAIR || TW == 2, "pairs of tiles");
  static_assert(TW == 1 ? NWV <= 32 : NWV <= 8, "per-wave visit counts packed in 32 bits");
  __shared__ __attribute__((aligned(1024))) uint8_t ring[kRing][STAGE];
  __shared__ float bias[kRing][NT];
  __shared__ unsigned long long Umask[32];
  __shared__ int Wpref[33];
  __shared__ uint16_t Blist[2048];
  __shared__ uint16_t Act[2048];
  __shared__ uint16_t Ord[2048];

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

  int tpos[TW], rpos[TW], rhead[TW];
  bool rvalid[TW];
#pragma unroll
  for (int u = 0; u < TW; ++u) {
    const int ti = TW * wv + u;
    tpos[u] = ti / tg.HT;
    rpos[u] = p0 + tpos[u];
    rhead[u] = (ti % tg.HT) * 16 + r;
    rvalid[u] = rpos[u] < pend;
  }
  // Q and dO operands (B of S^T = K Q^T and dP^T = V dO^T), the forward's LSE
  // and D = <dO, O> of the lane's head, in log2 units where they meet exp2
  bf16x8 qa[TW][KS], da[TW][KS];
  float lse2[TW], dlt[TW];
#pragma unroll
  for (int u = 0; u < TW; ++u) {
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

  const unsigned long long* mbase = mask + ((int64_t)h * T + si.start + p0) * W;
  const int nlist = ring_build_list<NWV, TW>(W, tg.HT, g.B == 128, mbase, npos, cdiag, Umask,
                                             Wpref, Blist, Act, Ord);
  const int sbl = g.B == 128 ? 1 : 0;
  const int nrouted = nlist << sbl;
  const int ndiag = (pend - cdiag * g.B + 63) / 64;
  const int NS = nrouted + ndiag;

  // ---- per-thread DMA sources: piece i of this thread is 16 bytes of K row
  // or V row kr of the block (a wave's pieces all K or all V), from the source
  // piece head_row_swz places at its slot
  const int64_t krs = (int64_t)g.Hkv * D * 2;  // bytes between consecutive keys
  const bool isk = wv * NP * 1024 < KBYTES;
  const uint8_t* rbase = (const uint8_t*)(isk ? p.k : p.v) + (si.start * (int64_t)g.Hkv + h) * D * 2;
  int prow[NP];
  const uint8_t* pbase[NP];
#pragma unroll
  for (int i = 0; i < NP; ++i) {
    const int o = ((wv * NP + i) * 1024 + lane * 16) % KBYTES;
    prow[i] = o / KROW;
    pbase[i] = rbase + prow[i] * krs + (((o % KROW) / 16) ^ head_row_swz<D>(prow[i])) * 16;
  }
  const int bpos = min(p0 + (TW * wv + min(lane, TW - 1)) / tg.HT, pend - 1);
  const float* bsrc = p.log_prior + ((int64_t)h * T + si.start + bpos) * g.C_slots;
  const int kmax = pend - 1;
  auto issue_at = [&](int key0, int c, uint32_t slot, uint32_t bslot) {
    if (key0 + 63 <= kmax) {
#pragma unroll
      for (int i = 0; i < NP; ++i)
        lds_dma16(pbase[i] + (int64_t)key0 * krs, slot + (wv * NP + i) * 1024);
    } else {
      // rows past the sequence end (its last chunk): the last key again
#pragma unroll
      for (int i = 0; i < NP; ++i)
        lds_dma16(pbase[i] + (int64_t)(min(key0 + prow[i], kmax) - prow[i]) * krs,
                  slot + (wv * NP + i) * 1024);
    }
    if (lane < TW) lds_dma4(bsrc + c, bslot + wv * TW * 4);
  };
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

  f32x4 o[TW][DT];
#pragma unroll
  for (int u = 0; u < TW; ++u)
#pragma unroll
    for (int dt = 0; dt < DT; ++dt) o[u][dt] = f32x4{0.f, 0.f, 0.f, 0.f};
  const float sl2 = p.scale * kLog2e;
  const int rsw = head_row_swz<D>(r);  // rows 16 t + r share r's swizzle
  int koff[KS];
#pragma unroll
  for (int ks = 0; ks < KS; ++ks) koff[ks] = r * KROW + ((4 * ks + gq) ^ rsw) * 16;
  // transposing reads: lane (gq, r) points at row 4 gq + r / 4 (+ 32 h2, + 16),
  // dims 16 dt + 4 (r % 4) .. +3, i.e. piece 2 dt + (r % 4) / 2 at its slot
  // ((2 dt) ^ f) + (r % 4) / 2 (f even), byte 8 (r % 2)
  const int trow = 4 * gq + (r >> 2);
  const int tb = trow * KROW + 16 * ((r & 3) >> 1) + 8 * (r & 1);
  const int tx = head_row_swz<D>(trow) >> 1;
  float* dbias = p.dbias;
  const uint32_t ring0 = lds_addr(&ring[0][0]), bias0 = lds_addr(&bias[0][0]);

  auto active_mask = [&](int j) -> uint32_t {
    const uint32_t act = Act[j];
    uint32_t am = 0;
#pragma unroll
    for (int u = 0; u < TW; ++u)
      am |= (rvalid[u] && ((act >> tpos[u]) & 1u)) ? (1u << u) : 0u;
    return am;
  };
  auto routed_step = [&](int st, lds_u8* kv, uint32_t am) {
    float bz[TW], ds[TW];
    const float* bs = &bias[st & 3][TW * wv];
#pragma unroll
    for (int u = 0; u < TW; ++u) {
      bz[u] = bs[u] * kLog2e;
      ds[u] = 0.f;
    }
    const int c = listed(st);
    static_for<0, (PAIR ? TW / 2 : TW)>([&](auto k_) {
      constexpr int U0 = PAIR ? 2 * decltype(k_)::value : decltype(k_)::value;
      constexpr int NTL = PAIR ? 2 : 1;
      if ((am >> U0) & 1u) {
        visit_dq<D, false, U0, NTL, TW>(kv, kv + KBYTES, koff, tb, tx, qa, da, lse2, dlt, o, ds,
                                        sl2, bz, 0, rpos);
        // the tile's sum of dS over the block's keys and its 16 heads
#pragma unroll
        for (int u = U0; u < U0 + NTL; ++u) {
          float d = row16_sum(ds[u]);
          d += xor16(d);
          d += xor32(d);
          if (lane == 0)
            atomicAdd(&dbias[((int64_t)h * T + si.start + rpos[u]) * g.C_slots + c], d);
        }
      }
    });
  };
  auto diag_step = [&](int st, lds_u8* kv) {
    float bz[TW], ds[TW];
#pragma unroll
    for (int u = 0; u < TW; ++u) {
      bz[u] = 0.f;
      ds[u] = 0.f;
    }
    const int key0 = cdiag * g.B + ((st - nrouted) << 6);
    static_for<0, (PAIR ? TW / 2 : TW)>([&](auto k_) {
      constexpr int U0 = PAIR ? 2 * decltype(k_)::value : decltype(k_)::value;
      constexpr int NTL = PAIR ? 2 : 1;
      if (rvalid[U0])
        visit_dq<D, true, U0, NTL, TW>(kv, kv + KBYTES, koff, tb, tx, qa, da, lse2, dlt, o, ds,
                                       sl2, bz, key0 + 4 * gq, rpos);
    });
  };
  __builtin_amdgcn_s_waitcnt(0 | (7 << 4));  // operand and mask reads done first
  if (sbl == 0) {
    // 64-key chunks: two blocks per barrier, the next two loading meanwhile
    // (the forward ring kernel's schedule)
    issue(0, ring0, bias0);
    if (NS > 1) issue(1, ring0 + STAGE, bias0 + 4 * NT);
    auto pair_enter = [&](int st) {
      if (st & 1) return;
      wait_vm<0>();
      asm volatile("" ::: "memory");
      __builtin_amdgcn_s_barrier();
      asm volatile("" ::: "memory");
#pragma unroll 1
      for (int b = st + 2; b < min(st + 4, NS); ++b)
        issue(b, ring0 + (b & 3) * STAGE, bias0 + (b & 3) * 4 * NT);
    };
    for (int st = 0; st < nrouted; ++st) {
      pair_enter(st);
      routed_step(st, (lds_u8*)&ring[st & 3][0], active_mask(st));
    }
    for (int st = nrouted; st < NS; ++st) {
      pair_enter(st);
      diag_step(st, (lds_u8*)&ring[st & 3][0]);
    }
  } else {
    // 128-key chunks: one block per barrier, three ahead; every step issues
    // exactly one block's loads (past the list's end the last block again,
    // into the free slot), so one fixed counted wait proves slot st & 3 done
    issue(0, ring0, bias0);
    issue(min(1, NS - 1), ring0 + STAGE, bias0 + 4 * NT);
    issue(min(2, NS - 1), ring0 + 2 * STAGE, bias0 + 8 * NT);
    auto enter = [&](int st) -> lds_u8* {
      wait_vm<2 * LPS>();
      asm volatile("" ::: "memory");
      __builtin_amdgcn_s_barrier();
      asm volatile("" ::: "memory");
      return (lds_u8*)&ring[st & 3][0];
    };
    auto leave = [&](int st, int cnext) {
      const int sr = st + 3, sx = min(sr, NS - 1);
      issue_at(block_key0(sx, cnext), cnext, ring0 + (sr & 3) * STAGE, bias0 + (sr & 3) * 4 * NT);
    };
    for (int st = 0; st < nrouted; ++st) {
      lds_u8* kv = enter(st);
      const int cnext = listed(min(st + 3, NS - 1));
      const uint32_t am = active_mask(st >> sbl);
      if (!am) leave(st, cnext);
      routed_step(st, kv, am);
      if (am) leave(st, cnext);
    }
    for (int st = nrouted; st < NS; ++st) {
      lds_u8* kv = enter(st);
      diag_step(st, kv);
      leave(st, 0);
    }
  }
  __builtin_amdgcn_s_waitcnt(0 | (7 << 4));  // no ring load outlives the kernel

  // dQ = s dQ^T^T, fp32: lane (gq, r) holds dims 16 dt + 4 gq .. +3 of head r
#pragma unroll
  for (int u = 0; u < TW; ++u) {
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

// Ring kernels (G >= 16): NT 16-row tiles per workgroup, so P = NT / (G / 16)
// positions.
static TileGeom make_ring_tiles(const Geom& g, int NT = kRingTiles, int TW = 2) {
  TileGeom t;
  t.TP = 1;
  t.HT = g.G / 16;
  t.NT = NT;
  t.TW = TW;
  t.P = t.NT / t.HT;
  t.tiles_per_seq = (g.max_seqlen + t.P - 1) / t.P;
  return t;
}

// varlen packs of at most this many sequences get a longest-first work list
constexpr int kScheduleMaxSeqs = 1024;

int64_t prefill_items_capacity(const Geom& g) {
  if (!g.cu_seqlens || g.num_seqs > kScheduleMaxSeqs || !(g.bf16 && g.G >= 16)) return 0;
  return (g.T + 7) / 8 + g.num_seqs;  // sum_s ceil(L_s / P) for any P >= 8
}

// Cost-sorted work list of a varlen pack (one workgroup of 1024 threads,
// num_seqs <= 1024).  A tile's cost grows with its first position (its rows
// see that many keys).  The sequences are taken longest first (by tile count,
// ties by index), and each sequence's tiles from its last (costliest) down to
// its first, so the grid ends on the short tiles of the short sequences while
// the workgroups running at any one time share one sequence's keys and
// values in the caches (interleaving sequences, or heads, by tile cost
// measured slower: the working set outgrows the L2).
//   n_s = ceil(L_s / P) tiles of sequence s; perm = sequences by n desc;
//   off_k = sum_{k' < k} n_perm[k']; entry off_k + j = (perm[k] << 16) |
//   (n_perm[k] - 1 - j); entries from sum_s n_s up to cap hold 0xffffffff.
__global__ __launch_bounds__(1024) void prefill_schedule_kernel(const int32_t* __restrict__ cu,
                                                                int num_seqs, int P,
                                                                uint32_t* __restrict__ items,
                                                                int64_t cap) {
  constexpr int NTH = 1024;
  __shared__ int nt[kScheduleMaxSeqs];         // tiles per sequence
  __shared__ int perm[kScheduleMaxSeqs];       // sequences by tile count, desc
  __shared__ int off[kScheduleMaxSeqs];        // first entry of each sorted sequence
  const int tid = threadIdx.x;
  for (int i = tid; i < num_seqs; i += NTH) nt[i] = (cu[i + 1] - cu[i] + P - 1) / P;
  __syncthreads();
  for (int i = tid; i < num_seqs; i += NTH) {
    const int n = nt[i];
    int rank = 0;
    for (int j = 0; j < num_seqs; ++j) {
      const int m = nt[j];
      rank += (m > n || (m == n && j < i)) ? 1 : 0;
    }
    perm[rank] = i;
  }
  __syncthreads();
  // exclusive prefix of the sorted counts (Hillis-Steele over <= 1024 entries)
  const int mine = tid < num_seqs ? nt[perm[tid]] : 0;
  off[tid] = mine;
  __syncthreads();
  for (int o = 1; o < NTH; o <<= 1) {
    const int y = tid >= o ? off[tid - o] : 0;
    __syncthreads();
    off[tid] += y;
    __syncthreads();
  }
  const int total = off[NTH - 1];
  const int first = off[tid] - mine;
  __syncthreads();
  off[tid] = first;
  __syncthreads();
  // entries: sorted sequence k's tiles, highest first (all threads share the
  // work of every sequence)
  for (int k = 0; k < num_seqs; ++k) {
    const int s = perm[k], n = nt[s], o = off[k];
    for (int j = tid; j < n; j += NTH)
      if (o + j < cap) items[o + j] = ((uint32_t)s << 16) | (uint32_t)(n - 1 - j);
  }
  for (int64_t i = total + tid; i < cap; i += NTH) items[i] = 0xffffffffu;
}

// The forward launch: eight waves of two tiles (four waves of eight tiles hold
// 384 of the 512 registers of a lane in Q and O alone at D = 128 and spill).
constexpr int kFwdTiles = 16, kFwdNFR = 2;
// tiles per wave of the forward ring kernel: 1 for groups of 16 heads, the
// two tiles of one position for groups of 32
static int rg_tw(const Geom& g) { return g.G == 32 ? 2 : 1; }

int prefill_positions_per_tile(const Geom& g) {
  return make_ring_tiles(g, kFwdTiles, rg_tw(g)).P;
}

hipError_t launch_prefill_schedule(const Geom& g, int P, uint32_t* items, int64_t cap,
                                   hipStream_t st) {
  hipLaunchKernelGGL(prefill_schedule_kernel, dim3(1), dim3(1024), 0, st, g.cu_seqlens,
                     g.num_seqs, P, items, cap);
  return hipGetLastError();
}

bool prefill_uses_ring(const Geom& g) { return g.bf16 && g.G >= 16; }

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
  // the forward's tiling: 16 waves of one tile (G = 16) or 8 of a pair (G = 32)
  const TileGeom rg = make_ring_tiles(g, 16, g.G == 32 ? 2 : 1);
  dim3 grid(rg.tiles_per_seq, g.num_seqs, g.Hkv);
#define DASH_BQ(DD, NW, TW_, PR) \
  hipLaunchKernelGGL((bwd_dq_ring_kernel<DD, NW, TW_, PR>), grid, dim3(64 * NW), 0, st, g, p, rg)
  if (g.G == 32) {
    if (g.D == 64) DASH_BQ(64, 8, 2, true); else DASH_BQ(128, 8, 2, true);
  } else {
    if (g.D == 64) DASH_BQ(64, 16, 1, false); else DASH_BQ(128, 16, 1, false);
  }
#undef DASH_BQ
  return hipGetLastError();
}

hipError_t launch_prefill_attn(const Geom& g, const PrefillParams& p, hipStream_t st) {
  if (g.T == 0) return hipSuccess;
  if (g.bf16) {
    const TileGeom tg = make_tiles(g);
    dim3 grid(tg.tiles_per_seq, g.num_seqs, g.Hkv);
    if (prefill_uses_ring(g)) {
      constexpr int NFR = kFwdNFR;
      const TileGeom rg = make_ring_tiles(g, kFwdTiles, rg_tw(g));
      const int64_t cap = prefill_items_capacity(g);
      const uint32_t* items = nullptr;
      int64_t nwork = (int64_t)rg.tiles_per_seq * g.num_seqs;
      if (cap > 0 && p.items) {
        hipError_t e = launch_prefill_schedule(g, rg.P, p.items, cap, st);
        if (e != hipSuccess) return e;
        items = p.items;
        nwork = cap;
      }
      dim3 rgrid((unsigned)nwork, g.Hkv);
      dim3 tgrid((g.max_seqlen + 63) / 64, g.num_seqs, g.Hkv);
  // groups of 16 heads: 16 waves of one tile each (four waves a SIMD to
  // overlap their visits; 15.9 -> 15.2 ms at 64K against 8 waves of two);
  // groups of 32: 8 waves, each the two tiles of one position
#define DASH_RING(DD, PAIR)                                                                 \
  do {                                                                                      \
    if (PAIR)                                                                               \
      hipLaunchKernelGGL((prefill_attn_ring_kernel<DD, 8, 2, true, NFR>), rgrid,            \
                         dim3(64 * 8), 0, st, g, p, rg, items);                             \
    else                                                                                    \
      hipLaunchKernelGGL((prefill_attn_ring_kernel<DD, 16, 1, false, NFR>), rgrid,          \
                         dim3(64 * 16), 0, st, g, p, rg, items);                            \
  } while (0)
      if (g.D == 64) {
        hipLaunchKernelGGL(vt_transpose_kernel<64>, tgrid, dim3(256), 0, st, g,
                           (const uint16_t*)p.v, (uint16_t*)p.vt, p.Tp);
        if (rg.HT == 2) DASH_RING(64, true); else DASH_RING(64, false);
      } else {
        hipLaunchKernelGGL(vt_transpose_kernel<128>, tgrid, dim3(256), 0, st, g,
                           (const uint16_t*)p.v, (uint16_t*)p.vt, p.Tp);
        if (rg.HT == 2) DASH_RING(128, true); else DASH_RING(128, false);
      }
#undef DASH_RING
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
