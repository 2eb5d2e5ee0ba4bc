// Phase 2, incremental decoding ("Fase 2" of the gist.science technical
// summary; the implementation bullet of its contributions names prefill and
// incremental decoding).  One new query per sequence attends to the active
// chunks of its cached K/V (the routing bias added before the softmax) and to
// its own, partial, diagonal chunk.  This is memory-bound: every active K/V
// byte is read once and used by only G query rows.
//
// Split-K: the work of one (sequence, KV head) is the list of its active
// chunks in order, cut into 64-key blocks, then the diagonal blocks.  The
// nsplit workgroups of that pair each take an equal share of the list by
// rank (counted from the popcounts of the mask words, so the split balances
// active work, not chunk ranges).  A workgroup streams its blocks through
// LDS (K row-major, V transposed; register prefetch of the next block); each
// of its 4 waves handles 16 of the 64 keys of every block with its own
// online-softmax state: S^T = K Q^T (16x16x32 bf16 MFMA), then
// O^T += V^T P^T (16x16x16 bf16 MFMA over the wave's 16 keys).  The waves
// merge in LDS and write an unnormalised partial (max, sum, acc) per split;
// the combine kernel merges the splits into O and LSE.
#include "attn_stage.h"
#include "dash_device.h"
#include "dash_internal.h"

namespace dash {

hipError_t launch_rowattn_f32_decode(const Geom& g, const PrefillParams& p,
                                     const int32_t* seqlens, int64_t batch, hipStream_t st);

// Two workgroups fit a CU (LDS).  The second launch-bounds argument is the
// minimum number of waves per SIMD (amdgpu_waves_per_eu), not CUDA's blocks
// per multiprocessor: with 256 threads a workgroup puts one wave on each of
// the four SIMDs, so 2 waves per SIMD is two workgroups per CU.  Groups of up
// to 32 heads keep their registers within that budget (the two-tile variant
// took 260 without it).
template <int D, int NT>
__global__ __launch_bounds__(256, NT <= 2 ? 2 : 1) void decode_attn_kernel(Geom g, DecodeParams p) {
  constexpr int NTH = 256;
  static_assert(NTH == 256, "two waves per SIMD means two workgroups per CU only at 256 threads");
  constexpr int kMaxDecodeTiles = NT;  // ceil(G / 16)
  const int ntile = NT;
  using C = StageCfg<D, NTH>;
  constexpr int KS = D / 32;
  constexpr int DT = D / 16;
  __shared__ __attribute__((aligned(16))) uint16_t Ks[2][C::KS_ELEMS];
  __shared__ __attribute__((aligned(16))) uint16_t Vt[2][C::VT_ELEMS];
  __shared__ int Wpref[33];
  __shared__ uint16_t Blist[2048];
  __shared__ float Mw[4][16], Lw[4][16];

  const int tid = threadIdx.x, lane = tid & 63, wv = tid >> 6;
  const int r = lane & 15, gq = lane >> 4;
  const int split = blockIdx.x, b = blockIdx.y, h = blockIdx.z;
  const int batch = gridDim.y;
  const int L = p.seqlens[b];
  const int i = L - 1;
  const int n = i / g.B;
  const int W = g.W;
  const int G = g.G;
  const int64_t base_row = (int64_t)b * g.max_seqlen;
  const unsigned long long* mrow =
      (const unsigned long long*)p.mask + ((int64_t)h * batch + b) * W;

  if (tid < 64) {
    const int cnt = (tid < W) ? __popcll(mrow[tid] & routable_bits(tid, n)) : 0;
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
    unsigned long long v = mrow[tid] & routable_bits(tid, n);
    int o = Wpref[tid];
    while (v) {
      Blist[o++] = (uint16_t)(tid * 64 + __ffsll(v) - 1);
      v &= v - 1;
    }
  }
  __syncthreads();
  const int SB = g.B / 64;
  const int nrouted = Wpref[W] * SB;
  const int ndiag = (i - n * g.B) / 64 + 1;
  const int N = nrouted + ndiag;
  const int it0 = (int)(((int64_t)N * split) / p.nsplit);
  const int it1 = (int)(((int64_t)N * (split + 1)) / p.nsplit);

  // Q operands; a tile's row r is query head 16u + r of the group
  bf16x8 qa[kMaxDecodeTiles][KS];
  bool rvalid[kMaxDecodeTiles];
#pragma unroll
  for (int u = 0; u < kMaxDecodeTiles; ++u) {
    const int head = 16 * u + r;
    rvalid[u] = (u < ntile) && (head < G);
    const int64_t qrow = ((int64_t)b * g.Hq + h * G + head) * D;
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) {
      u32x4 v = {0u, 0u, 0u, 0u};
      if (rvalid[u]) v = ldg16((const uint16_t*)p.q + qrow + 32 * ks + 8 * gq);
      qa[u][ks] = as_bf16x8(v);
    }
  }
  f32x4 o[kMaxDecodeTiles][DT];
  float m[kMaxDecodeTiles], l[kMaxDecodeTiles];
#pragma unroll
  for (int u = 0; u < kMaxDecodeTiles; ++u) {
    m[u] = -INFINITY;
    l[u] = 0.f;
#pragma unroll
    for (int dt = 0; dt < DT; ++dt) o[u][dt] = f32x4{0.f, 0.f, 0.f, 0.f};
  }
  const float sl2 = p.scale * kLog2e;
  const float* lrow = p.log_prior + ((int64_t)h * batch + b) * g.C_slots;
  const uint16_t* kp = (const uint16_t*)p.k;
  const uint16_t* vp = (const uint16_t*)p.v;

  auto stage_key0 = [&](int st, int& c, bool& diag) -> int {
    if (st < nrouted) {
      c = Blist[st / SB];
      diag = false;
      return c * g.B + (st % SB) * 64;
    }
    c = n;
    diag = true;
    return n * g.B + (st - nrouted) * 64;
  };
  StageRegs<D, NTH> R;
  if (it0 < it1) {
    int c0;
    bool d0;
    const int k0 = stage_key0(it0, c0, d0);
    stage_load<D, NTH>(R, kp, vp, base_row, k0, d0 ? L : g.max_seqlen, g.Hkv, h, tid);
  }
  for (int st = it0; st < it1; ++st) {
    const int buf = (st - it0) & 1;
    int c;
    bool diag;
    const int key0 = stage_key0(st, c, diag);
    stage_store<D, NTH>(R, Ks[buf], Vt[buf], tid);
    __syncthreads();
    if (st + 1 < it1) {
      int c1;
      bool d1;
      const int k1 = stage_key0(st + 1, c1, d1);
      stage_load<D, NTH>(R, kp, vp, base_row, k1, d1 ? L : g.max_seqlen, g.Hkv, h, tid);
    }
    const float bias = diag ? 0.f : lrow[c] * kLog2e;
    const uint16_t* ks_ = Ks[buf];
    const uint16_t* vt_ = Vt[buf];
    // this wave's keys: 16*wv + 4*gq + j
    const int vcol = vt_col(16 * wv + 4 * gq);
#pragma unroll
    for (int u = 0; u < kMaxDecodeTiles; ++u) {
      if (u >= ntile) break;
      f32x4 sacc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int ks = 0; ks < KS; ++ks) {
        const bf16x8 ak = as_bf16x8(
            *reinterpret_cast<const u32x4*>(ks_ + (16 * wv + r) * C::KSTR + 32 * ks + 8 * gq));
        sacc = mfma16x16x32(ak, qa[u][ks], sacc);
      }
      float zmax = -INFINITY;
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        float z = sacc[j] * sl2 + bias;
        bool ok = rvalid[u];
        if (diag) ok = ok && (key0 + 16 * wv + 4 * gq + j <= i);
        z = ok ? z : -INFINITY;
        sacc[j] = z;
        zmax = fmaxf(zmax, z);
      }
      zmax = fmaxf(zmax, __shfl_xor(zmax, 16));
      zmax = fmaxf(zmax, __shfl_xor(zmax, 32));
      const float mnew = fmaxf(m[u], zmax);
      const float muse = (mnew == -INFINITY) ? 0.f : mnew;
      const float alpha = exp2f(m[u] - muse);
      const float p0 = exp2f(sacc[0] - muse), p1 = exp2f(sacc[1] - muse);
      const float p2 = exp2f(sacc[2] - muse), p3 = exp2f(sacc[3] - muse);
      l[u] = l[u] * alpha + ((p0 + p1) + (p2 + p3));
      m[u] = mnew;
      const u32x2 pb = {pack_bf16x2(p0, p1), pack_bf16x2(p2, p3)};
#pragma unroll
      for (int dt = 0; dt < DT; ++dt) {
        o[u][dt] *= alpha;
        const u32x2 av = *reinterpret_cast<const u32x2*>(vt_ + (16 * dt + r) * C::VSTR + vcol);
        o[u][dt] = mfma16x16x16(as_s16x4(av), as_s16x4(pb), o[u][dt]);
      }
    }
  }
  __syncthreads();  // LDS staging buffers are reused for the merge below

  // ---- merge the 4 waves and write this split's partial
  float* Ow = reinterpret_cast<float*>(&Ks[0][0]);  // [4][16][D] floats fit in Ks+Vt
  // partials are [batch, Hkv, G, nsplit, *]: one query head's splits are contiguous
  const int64_t pbase = ((int64_t)b * g.Hkv + h) * G;
#pragma unroll
  for (int u = 0; u < kMaxDecodeTiles; ++u) {
    if (u >= ntile) break;
    float lt = l[u];
    lt += __shfl_xor(lt, 16);
    lt += __shfl_xor(lt, 32);
    if (gq == 0) {
      Mw[wv][r] = m[u];
      Lw[wv][r] = lt;
    }
#pragma unroll
    for (int dt = 0; dt < DT; ++dt)
#pragma unroll
      for (int j = 0; j < 4; ++j) Ow[(wv * 16 + r) * D + 16 * dt + 4 * gq + j] = o[u][dt][j];
    __syncthreads();
    for (int idx = tid; idx < 16 * D; idx += 256) {
      const int row = idx / D, d = idx - row * D;
      const int head = 16 * u + row;
      if (head >= G) continue;
      float M = -INFINITY;
#pragma unroll
      for (int w = 0; w < 4; ++w) M = fmaxf(M, Mw[w][row]);
      const float Mu = (M == -INFINITY) ? 0.f : M;
      float acc = 0.f, ls = 0.f;
#pragma unroll
      for (int w = 0; w < 4; ++w) {
        const float sc = exp2f(Mw[w][row] - Mu);
        acc += Ow[(w * 16 + row) * D + d] * sc;
        ls += Lw[w][row] * sc;
      }
      const int64_t pr = (pbase + head) * p.nsplit + split;
      p.part_acc[pr * D + d] = acc;
      if (d == 0) {
        p.part_ml[pr * 2 + 0] = M;
        p.part_ml[pr * 2 + 1] = ls;
      }
    }
    __syncthreads();
  }
}

// One workgroup per (query head, sequence, KV head).  The head's nsplit
// partials are contiguous, so every load of the merge is issued in one round:
// the (max, sum) pairs into LDS, each thread's accumulator pieces (4 dims of
// some splits) into registers.  Each thread scales and adds its pieces, the
// split groups are added in LDS, and D threads write the output.
template <int D>
__global__ __launch_bounds__(256) void decode_combine_kernel(Geom g, DecodeParams p) {
  constexpr int NTH = 256;
  constexpr int TPR = D / 4;        // threads per split row (4 dims each)
  constexpr int SG = NTH / TPR;     // split groups handled side by side
  constexpr int MAXS = 64;          // most splits decode_num_splits hands out
  constexpr int PPT = MAXS / SG;    // split rows per thread
  __shared__ float Sm[MAXS], Sl[MAXS];
  __shared__ float Part[SG][D];
  const int q = blockIdx.x, b = blockIdx.y, h = blockIdx.z;
  const int batch = gridDim.y;
  const int tid = threadIdx.x;
  const int G = g.G;
  const int ns = p.nsplit;
  const int64_t row0 = (((int64_t)b * g.Hkv + h) * G + q) * ns;  // first split row
  const int sg = tid / TPR, d0 = (tid % TPR) * 4;
  f32x4 x[PPT];
#pragma unroll
  for (int k = 0; k < PPT; ++k) {
    const int sp = sg + SG * k;
    x[k] = sp < ns ? *reinterpret_cast<const f32x4*>(p.part_acc + (row0 + sp) * D + d0)
                   : f32x4{0.f, 0.f, 0.f, 0.f};
  }
  if (tid < MAXS) {
    Sm[tid] = tid < ns ? p.part_ml[(row0 + tid) * 2] : -INFINITY;
    Sl[tid] = tid < ns ? p.part_ml[(row0 + tid) * 2 + 1] : 0.f;
  }
  __syncthreads();
  float M = -INFINITY;
  for (int sp = 0; sp < ns; ++sp) M = fmaxf(M, Sm[sp]);
  f32x4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
  for (int k = 0; k < PPT; ++k) {
    const int sp = sg + SG * k;
    if (sp < ns && Sm[sp] != -INFINITY) acc += x[k] * exp2f(Sm[sp] - M);
  }
  *reinterpret_cast<f32x4*>(&Part[sg][d0]) = acc;
  __syncthreads();
  if (tid < D) {
    float v = 0.f;
#pragma unroll
    for (int k = 0; k < SG; ++k) v += Part[k][tid];
    float ls = 0.f;
    for (int sp = 0; sp < ns; ++sp)
      if (Sm[sp] != -INFINITY) ls += Sl[sp] * exp2f(Sm[sp] - M);
    v /= ls;
    const int64_t orow = ((int64_t)b * g.Hq + h * G + q) * D;
    if (g.bf16)
      ((uint16_t*)p.out)[orow + tid] = (uint16_t)f32_to_bf16(v);
    else
      ((float*)p.out)[orow + tid] = v;
    if (p.lse && tid == 0) p.lse[(int64_t)(h * G + q) * batch + b] = (M + __log2f(ls)) * kLn2;
  }
}

int decode_num_splits(const Geom& g) {
  const int pairs = g.num_seqs * g.Hkv;
  // about 512 workgroups: two fit a CU (LDS), so on 256 CUs every split
  // runs in one round (16 x 128K: 512 -> 142 us per step, 1024 -> 149 us,
  // 2048 -> 172 us)
  int ns = (512 + pairs - 1) / max(pairs, 1);
  ns = max(1, min(ns, 64));  // the combine holds at most 64 splits
  // never more splits than 64-key blocks a sequence can have
  const int maxblocks = (g.max_seqlen + 63) / 64;
  return max(1, min(ns, maxblocks));
}

hipError_t launch_decode_attn(const Geom& g, const DecodeParams& p, hipStream_t st) {
  if (g.num_seqs == 0) return hipSuccess;
  if (!g.bf16) {
    PrefillParams pp;
    pp.q = p.q;
    pp.k = p.k;
    pp.v = p.v;
    pp.mask = p.mask;
    pp.log_prior = p.log_prior;
    pp.out = p.out;
    pp.lse = p.lse;
    pp.scale = p.scale;
    return launch_rowattn_f32_decode(g, pp, p.seqlens, g.num_seqs, st);
  }
  const int ntile = (g.G + 15) / 16;
  dim3 grid(p.nsplit, g.num_seqs, g.Hkv);
#define DASH_DEC(DD, NTV) \
  hipLaunchKernelGGL((decode_attn_kernel<DD, NTV>), grid, dim3(256), 0, st, g, p)
#define DASH_DEC_NT(DD)                         \
  do {                                          \
    if (ntile == 1) DASH_DEC(DD, 1);            \
    else if (ntile == 2) DASH_DEC(DD, 2);       \
    else DASH_DEC(DD, 4);                       \
  } while (0)
  if (g.D == 64) {
    DASH_DEC_NT(64);
    hipLaunchKernelGGL(decode_combine_kernel<64>, dim3(g.G, g.num_seqs, g.Hkv), dim3(256), 0, st,
                       g, p);
  } else {
    DASH_DEC_NT(128);
    hipLaunchKernelGGL(decode_combine_kernel<128>, dim3(g.G, g.num_seqs, g.Hkv), dim3(256), 0,
                       st, g, p);
  }
#undef DASH_DEC_NT
#undef DASH_DEC
  return hipGetLastError();
}

}  // namespace dash
