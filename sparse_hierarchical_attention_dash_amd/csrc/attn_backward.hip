// Backward of phase 2 for the keys and values, and the per-row terms the
// backward needs ("Fase 2: Prior-Geinduceerde Spaarzame Softmax" of the
// gist.science technical summary; the pages rest the method on its being
// differentiable end to end, "Fase 1", Differentieerbaarheid bullet).
//
//   D_i   = <dO_i, O_i>                                  (bwd_delta_kernel)
//   dV_j  = sum_i P_ij dO_i,   dK_j = s sum_i dS_ij q_i  (bwd_dkdv_kernel)
//   with P_ij = exp(s <q_i, k_j> + b_ij - LSE_i) from the forward's LSE and
//   dS_ij = P_ij (<dO_i, v_j> - D_i), over every query row i that sees key j:
//   the rows that have j's chunk active (bias b = log_prior) and the rows of
//   j's own chunk at or after j (bias 0).
//
// bwd_headt_kernel: Q and dO copied per (token, KV head) as contiguous blocks
// of their transposes (units of two dims x four heads).
// bwd_dkdv_kernel: one workgroup of 4 waves per (64-key block, slice of 4096
// rows, sequence, KV head); wave w owns keys 16w .. 16w+15 of the block and
// holds their K and V rows as MFMA operands for the whole kernel.  It scans
// its slice's mask words 1024 rows at a time, compacts the rows that see the
// block (ballots and a block-wide prefix, in row order), and streams those
// rows through a ring of LDS stages filled by direct global->LDS loads (q_i
// and dO_i XOR-swizzled, their transposes in the unit order of
// bwd_headt_kernel, so that the operand reads below are free of bank
// conflicts; the row's LSE, D and bias beside them), several rows ahead of
// the one computed:
//   S  = Q_i K_w^T and dP = dO_i V_w^T   (16 heads x 16 keys, 16x16x32 MFMA;
//                                         the accumulators of S are exactly
//                                         the operand layout P needs below)
//   P  = exp2(s S + b - LSE),  dS = P (dP - D)
//   dV_w^T += dO_i^T P,  dK_w^T += Q_i^T dS   (16x16x16 MFMA over the heads)
// The slices of a block add their sums into the zeroed fp32 dK and dV by
// atomics: a block that most rows route to (an early or planted chunk) would
// otherwise hold one workgroup for the whole sequence.
// The group's heads go in tiles of 16 (G = 16 or 32).
#include "dash_device.h"
#include "dash_internal.h"

namespace dash {

// D_i = <dO_i, O_i> per (query head, token): one thread per (token, head).
template <int D>
__global__ __launch_bounds__(256) void bwd_delta_kernel(Geom g, const uint16_t* __restrict__ out,
                                                        const uint16_t* __restrict__ dout,
                                                        float* __restrict__ delta) {
  const int64_t idx = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (idx >= g.T * g.Hq) return;
  const int64_t t = idx / g.Hq;
  const int qh = (int)(idx - t * g.Hq);
  const uint16_t* o = out + idx * D;
  const uint16_t* d = dout + idx * D;
  float acc = 0.f;
#pragma unroll 4
  for (int e = 0; e < D; e += 8) {
    const u32x4 a = ldg16(o + e), b = ldg16(d + e);
#pragma unroll
    for (int w = 0; w < 4; ++w) {
      acc = fmaf(bf16lo(a[w]), bf16lo(b[w]), acc);
      acc = fmaf(bf16hi(a[w]), bf16hi(b[w]), acc);
    }
  }
  delta[(int64_t)qh * g.T + t] = acc;
}

__global__ __launch_bounds__(256) void zero_kernel(float* __restrict__ x, int64_t n) {
  const int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (i < n) x[i] = 0.f;
}

constexpr int kDkdvSlice = 4096;  // rows per workgroup of bwd_dkdv_kernel
constexpr int kDkdvTiles = 1;     // 16-key tiles per wave of bwd_dkdv_kernel (2: slower)

// The transposed copy of one (token, KV head): 16-byte units of two adjacent
// dims x four heads, unit (quad, pair) at (quad D/2 + pair) 16 bytes,
//   xt[(h T + t) G D + 8 (quad D/2 + pair) + 4 parity + jj]
//     = x[t, h G + 4 quad + jj, 2 pair + parity],
// so that the 16 lanes of an MFMA operand read (16 consecutive dims, one
// head quad, 8 bytes each) cover one contiguous 128 bytes of LDS.
template <int D, int G>
__global__ __launch_bounds__(256) void bwd_headt_kernel(Geom g, const uint16_t* __restrict__ x,
                                                        uint16_t* __restrict__ xt) {
  constexpr int ROW = D + 8;
  constexpr int NU = G * D / 8;  // 16-byte units
  __shared__ __align__(16) uint16_t tile[G * ROW];
  const int64_t tok = blockIdx.x;
  const int h = blockIdx.y, tid = threadIdx.x;
  for (int u = tid; u < NU; u += 256) {
    const int j = u / (D / 8), d0 = (u % (D / 8)) * 8;
    *reinterpret_cast<u32x4*>(&tile[j * ROW + d0]) =
        ldg16(x + (tok * g.Hq + h * G + j) * (int64_t)D + d0);
  }
  __syncthreads();
  uint16_t* dst = xt + ((int64_t)h * g.T + tok) * (D * G);
  for (int u = tid; u < NU; u += 256) {
    const int quad = u / (D / 2), pair = u % (D / 2);
    u32x4 o;
#pragma unroll
    for (int w = 0; w < 4; ++w) {
      const int par = w >> 1, jj = 2 * (w & 1);
      const int d = 2 * pair + par, j = 4 * quad + jj;
      o[w] = (uint32_t)tile[j * ROW + d] | ((uint32_t)tile[(j + 1) * ROW + d] << 16);
    }
    *reinterpret_cast<u32x4*>(dst + 8 * u) = o;
  }
}

template <int D, int HT, int KT>
struct DkdvCfg {
  static constexpr int NW = 4 / KT;                    // waves: KT 16-key tiles each
  static constexpr int NTH = 64 * NW;
  static constexpr int G = 16 * HT;
  static constexpr int NS = HT == 1 ? 4 : 3;           // ring stages, one row each
  static constexpr int ABYTES = G * D * 2;             // one array of one row
  static constexpr int SBYTES = 4 * ABYTES;            // Q, dO, Q^T, dO^T
  static constexpr int AU = ABYTES / 16;               // 16-byte units per array
  static constexpr int NUT = 4 * AU / NTH;             // unit loads per thread per stage
  static constexpr int PER = NUT + 2;                  // loads per wave per stage
  static_assert(4 * AU % NTH == 0, "units per stage");
};

template <int D, int HT, int KT>
__global__ __launch_bounds__(256 / KT) void bwd_dkdv_kernel(Geom g, BwdParams p, float* dk,
                                                            float* dv) {
  using C = DkdvCfg<D, HT, KT>;
  static_assert(C::NTH == 256 / KT, "launch bounds");
  constexpr int G = C::G;
  constexpr int KS = D / 32;
  constexpr int DT = D / 16;
  constexpr int NS = C::NS;
  constexpr int NTH = C::NTH;
  constexpr int NW = C::NW;
  constexpr int UPH = D / 8;      // units per head row of Q / dO
  constexpr int NR = 1024;        // rows scanned per compaction
  __shared__ __align__(16) uint8_t Ring[NS * C::SBYTES];
  __shared__ __align__(16) float Sc[NS][NW][64];  // per wave: LSE (lanes < G), D (G .. 2G-1)
  __shared__ __align__(16) float Bz[NS][NW][4];   // per wave: the row's bias
  __shared__ int Rows[NR];
  __shared__ int Wcnt[NR / NTH][NW];

  const int tid = threadIdx.x, lane = tid & 63, wv = tid >> 6;
  const int r = lane & 15, gq = lane >> 4;
  const int blk = blockIdx.x, s = blockIdx.z / g.Hkv, h = blockIdx.z % g.Hkv;
  const SeqInfo si = seq_info(g.cu_seqlens, nullptr, s, g.max_seqlen, g.B);
  const int key0 = blk * 64;
  if (key0 >= si.len) return;
  // this workgroup's slice of the rows that may see the block
  const int rlo = max(key0, (int)blockIdx.y * kDkdvSlice);
  const int rhi = min(si.len, ((int)blockIdx.y + 1) * kDkdvSlice);
  if (rlo >= rhi) return;
  const int c = key0 / g.B;            // the block's chunk
  const int cend = min((c + 1) * g.B, si.len);
  const int kmax = si.len - 1;
  const int64_t T = g.T;
  const unsigned long long* __restrict__ mask = (const unsigned long long*)p.mask;

  // this wave's KT tiles of 16 keys: K and V rows as the B operand of Q K^T
  // and dO V^T
  int mykey[KT];
  bf16x8 kf[KT][KS], vf[KT][KS];
#pragma unroll
  for (int kt = 0; kt < KT; ++kt) {
    mykey[kt] = key0 + 16 * (KT * wv + kt) + r;
    const int64_t row = ((si.start + min(mykey[kt], kmax)) * g.Hkv + h) * (int64_t)D;
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) {
      kf[kt][ks] = as_bf16x8(ldg16((const uint16_t*)p.k + row + 32 * ks + 8 * gq));
      vf[kt][ks] = as_bf16x8(ldg16((const uint16_t*)p.v + row + 32 * ks + 8 * gq));
    }
  }
  // the operand loads complete here, so that the compiler's own waits for them
  // do not land inside the ring loop, where they would also wait for the ring
  wait_vm<0>();
  f32x4 adk[KT][DT], adv[KT][DT];
#pragma unroll
  for (int kt = 0; kt < KT; ++kt)
#pragma unroll
    for (int dt = 0; dt < DT; ++dt) {
      adk[kt][dt] = f32x4{0.f, 0.f, 0.f, 0.f};
      adv[kt][dt] = f32x4{0.f, 0.f, 0.f, 0.f};
    }
  const float sl2 = p.scale * kLog2e;
  const uint16_t* qg = (const uint16_t*)p.q;
  const uint16_t* dg = (const uint16_t*)p.dout;
  const uint16_t* qtg = (const uint16_t*)p.qt;
  const uint16_t* dtg = (const uint16_t*)p.dot;

  // one row into ring slot `slot`: thread tid loads units tid + 256 e
  auto issue = [&](int row, int slot) {
    const int64_t tok = si.start + row;
    const uint32_t base = lds_addr(Ring) + (uint32_t)(slot * C::SBYTES);
#pragma unroll
    for (int e = 0; e < C::NUT; ++e) {
      const int U = tid + NTH * e;
      const int arr = U / C::AU, u = U % C::AU;
      const uint16_t* src;
      if (arr < 2) {
        // row-major: head j, 16-byte piece (u % UPH) ^ (j % UPH)
        const int j = u / UPH, pc = (u % UPH) ^ (j % UPH);
        src = (arr == 0 ? qg : dg) + (tok * g.Hq + h * G + j) * (int64_t)D + 8 * pc;
      } else {
        // transposed: the units in their order (see bwd_headt_kernel)
        src = (arr == 2 ? qtg : dtg) + ((int64_t)h * T + tok) * (D * G) + 8 * u;
      }
      lds_dma16(src, __builtin_amdgcn_readfirstlane(base + (uint32_t)(16 * (NTH * e + 64 * wv))));
    }
    if (lane < 2 * G) {
      const float* src = lane < G ? p.lse + (int64_t)(h * G + lane) * T + tok
                                  : p.delta + (int64_t)(h * G + lane - G) * T + tok;
      lds_dma4(src, __builtin_amdgcn_readfirstlane(lds_addr(&Sc[slot][wv][0])));
    }
    if (lane == 0)  // the bias (any valid word for rows of the block's own chunk)
      lds_dma4(p.log_prior + ((int64_t)h * T + tok) * g.C_slots + c,
               __builtin_amdgcn_readfirstlane(lds_addr(&Bz[slot][wv][0])));
  };

  auto compute = [&](int slot, int row) {
    const uint8_t* st = Ring + slot * C::SBYTES;
    lds_u8* Qs = (lds_u8*)(st);
    lds_u8* Ds = (lds_u8*)(st + C::ABYTES);
    lds_u8* Qt = (lds_u8*)(st + 2 * C::ABYTES);
    lds_u8* Dt = (lds_u8*)(st + 3 * C::ABYTES);
    const bool own = row < cend;  // the block's own chunk: keys after the row are unseen
    const float bz = own ? 0.f : Bz[slot][wv][0] * kLog2e;
#pragma unroll
    for (int ht = 0; ht < HT; ++ht) {
      f32x4 sacc[KT], pacc[KT];
#pragma unroll
      for (int kt = 0; kt < KT; ++kt) {
        sacc[kt] = f32x4{0.f, 0.f, 0.f, 0.f};
        pacc[kt] = f32x4{0.f, 0.f, 0.f, 0.f};
      }
      const int j = 16 * ht + r;
#pragma unroll
      for (int ks = 0; ks < KS; ++ks) {
        // one read of the row's Q and dO fragments serves the wave's KT key tiles
        const int off = 16 * (j * UPH + ((4 * ks + gq) ^ (j % UPH)));
        const bf16x8 qf = as_bf16x8(lds_read16(Qs + off)), df = as_bf16x8(lds_read16(Ds + off));
#pragma unroll
        for (int kt = 0; kt < KT; ++kt) {
          sacc[kt] = mfma16x16x32(qf, kf[kt][ks], sacc[kt]);
          pacc[kt] = mfma16x16x32(df, vf[kt][ks], pacc[kt]);
        }
      }
      // lane (gq, r): heads 16 ht + 4 gq + j, key mykey[kt]
      u32x2 pb[KT], sb[KT];
#pragma unroll
      for (int kt = 0; kt < KT; ++kt) {
        float pv[4], ds[4];
#pragma unroll
        for (int jj = 0; jj < 4; ++jj) {
          const int hh = 16 * ht + 4 * gq + jj;
          float e = __builtin_amdgcn_exp2f(fmaf(sacc[kt][jj], sl2, bz - Sc[slot][wv][hh] * kLog2e));
          if (own) e = mykey[kt] <= row ? e : 0.f;
          e = mykey[kt] <= kmax ? e : 0.f;
          pv[jj] = e;
          ds[jj] = e * (pacc[kt][jj] - Sc[slot][wv][G + hh]);
        }
        pb[kt] = u32x2{cvt_pk_bf16(pv[0], pv[1]), cvt_pk_bf16(pv[2], pv[3])};
        sb[kt] = u32x2{cvt_pk_bf16(ds[0], ds[1]), cvt_pk_bf16(ds[2], ds[3])};
      }
      const int quad = 4 * ht + gq;
#pragma unroll
      for (int dt = 0; dt < DT; ++dt) {
        // A = X^T tile: dims 16 dt + r, heads 16 ht + 4 gq .. +3 (one read for
        // the KT key tiles)
        const int off = 16 * (quad * (D / 2) + 8 * dt + (r >> 1)) + 8 * (r & 1);
        typedef const __attribute__((address_space(3))) u32x2 lds_u32x2;
        const u32x2 ta = *reinterpret_cast<lds_u32x2*>(Dt + off);
        const u32x2 tq = *reinterpret_cast<lds_u32x2*>(Qt + off);
#pragma unroll
        for (int kt = 0; kt < KT; ++kt) {
          adv[kt][dt] = mfma16x16x16(as_s16x4(ta), as_s16x4(pb[kt]), adv[kt][dt]);
          adk[kt][dt] = mfma16x16x16(as_s16x4(tq), as_s16x4(sb[kt]), adk[kt][dt]);
        }
      }
    }
  };

  int seen = 0;  // rows this workgroup visited
  for (int r0 = rlo; r0 < rhi; r0 += NR) {
    // ---- rows r0 .. r0+1023 that see the block, compacted in order
    constexpr int NQ = NR / NTH;
    bool on[NQ];
    uint64_t bal[NQ];
    unsigned long long mw[NQ];
#pragma unroll
    for (int q = 0; q < NQ; ++q) {  // the mask words first, all in flight
      const int i = r0 + NTH * q + tid;
      mw[q] = i >= cend && i < rhi ? mask[((int64_t)h * T + si.start + i) * g.W + (c >> 6)] : 0ull;
    }
#pragma unroll
    for (int q = 0; q < NQ; ++q) {
      const int i = r0 + NTH * q + tid;
      // the block's own chunk: causal (i >= key0 here); later rows: the mask
      on[q] = i < rhi && (i < cend || ((mw[q] >> (c & 63)) & 1ull));
      bal[q] = __ballot(on[q]);
      if (lane == 0) Wcnt[q][wv] = __popcll(bal[q]);
    }
    __syncthreads();
    int total = 0;
#pragma unroll
    for (int q = 0; q < NQ; ++q) {
      int before = total;
#pragma unroll
      for (int w = 0; w < NW; ++w) {
        before += w < wv ? Wcnt[q][w] : 0;
        total += Wcnt[q][w];
      }
      if (on[q]) Rows[before + __popcll(bal[q] & ((1ull << lane) - 1ull))] = r0 + NTH * q + tid;
    }
    __syncthreads();
    seen += total;

    for (int k = 0; k < NS - 1 && k < total; ++k) issue(Rows[k], k);
    for (int k = 0; k < total; ++k) {
      // this wave's loads of row k have landed once at most the later
      // stages' loads are outstanding; the barrier then covers every wave's
      const int ahead = min(NS - 2, total - 1 - k);
      if (ahead >= 2) wait_vm<2 * C::PER>();
      else if (ahead == 1) wait_vm<C::PER>();
      else wait_vm<0>();
      __syncthreads();
      if (k + NS - 1 < total) issue(Rows[k + NS - 1], (k + NS - 1) % NS);
      compute(k % NS, Rows[k]);
    }
    __syncthreads();  // the ring and Rows are refilled
  }
  // ---- add this slice's sums for the wave's keys: lane (gq, r) holds dims
  // 16 dt + 4 gq .. +3 of key mykey
#pragma unroll
  for (int kt = 0; kt < KT; ++kt) {
    if (seen > 0 && mykey[kt] <= kmax) {
      const int64_t row = ((si.start + mykey[kt]) * g.Hkv + h) * (int64_t)D;
#pragma unroll
      for (int dt = 0; dt < DT; ++dt) {
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          atomicAdd(dk + row + 16 * dt + 4 * gq + j, adk[kt][dt][j] * p.scale);
          atomicAdd(dv + row + 16 * dt + 4 * gq + j, adv[kt][dt][j]);
        }
      }
    }
  }
}

// fp32 -> the storage dtype (bf16), n elements, 4 per thread
__global__ __launch_bounds__(256) void to_bf16_kernel(const float* __restrict__ src,
                                                      uint16_t* __restrict__ dst, int64_t n) {
  const int64_t i = ((int64_t)blockIdx.x * 256 + threadIdx.x) * 4;
  if (i >= n) return;
  const f32x4 v = *reinterpret_cast<const f32x4*>(src + i);
  const u32x2 w = {pack_bf16x2(v[0], v[1]), pack_bf16x2(v[2], v[3])};
  *reinterpret_cast<u32x2*>(dst + i) = w;
}

hipError_t launch_bwd_delta(const Geom& g, const void* out, const void* dout, float* delta,
                            hipStream_t st) {
  const int64_t n = g.T * g.Hq;
  if (n == 0) return hipSuccess;
  dim3 grid((unsigned)((n + 255) / 256));
  if (g.D == 64)
    hipLaunchKernelGGL(bwd_delta_kernel<64>, grid, dim3(256), 0, st, g, (const uint16_t*)out,
                       (const uint16_t*)dout, delta);
  else
    hipLaunchKernelGGL(bwd_delta_kernel<128>, grid, dim3(256), 0, st, g, (const uint16_t*)out,
                       (const uint16_t*)dout, delta);
  return hipGetLastError();
}

hipError_t launch_bwd_headt(const Geom& g, const void* x, void* xt, hipStream_t st) {
  if (g.T == 0) return hipSuccess;
  dim3 grid((unsigned)g.T, g.Hkv);
#define DASH_HT(DD, GG) \
  hipLaunchKernelGGL((bwd_headt_kernel<DD, GG>), grid, dim3(256), 0, st, g, (const uint16_t*)x, (uint16_t*)xt)
  if (g.G == 16) {
    if (g.D == 64) DASH_HT(64, 16); else DASH_HT(128, 16);
  } else {
    if (g.D == 64) DASH_HT(64, 32); else DASH_HT(128, 32);
  }
#undef DASH_HT
  return hipGetLastError();
}

hipError_t launch_bwd_dkdv(const Geom& g, const BwdParams& p, float* dk, float* dv,
                           hipStream_t st) {
  if (g.T == 0) return hipSuccess;
  // the row slices of a key block meet by atomics in the zeroed outputs
  const int64_t n = g.T * g.Hkv * g.D;
  hipLaunchKernelGGL(zero_kernel, dim3((unsigned)((n + 255) / 256)), dim3(256), 0, st, dk, n);
  hipLaunchKernelGGL(zero_kernel, dim3((unsigned)((n + 255) / 256)), dim3(256), 0, st, dv, n);
  dim3 grid((g.max_seqlen + 63) / 64, (g.max_seqlen + kDkdvSlice - 1) / kDkdvSlice,
            g.num_seqs * g.Hkv);
#define DASH_BK(DD, HH)                                                              \
  hipLaunchKernelGGL((bwd_dkdv_kernel<DD, HH, kDkdvTiles>), grid,                      \
                     dim3(DkdvCfg<DD, HH, kDkdvTiles>::NTH), 0, st, g, p, dk, dv)
  if (g.G == 16) {
    if (g.D == 64) DASH_BK(64, 1); else DASH_BK(128, 1);
  } else {
    if (g.D == 64) DASH_BK(64, 2); else DASH_BK(128, 2);
  }
#undef DASH_BK
  return hipGetLastError();
}

hipError_t launch_zero(float* x, int64_t n, hipStream_t st) {
  if (n == 0) return hipSuccess;
  hipLaunchKernelGGL(zero_kernel, dim3((unsigned)((n + 255) / 256)), dim3(256), 0, st, x, n);
  return hipGetLastError();
}

hipError_t launch_to_bf16(const float* src, void* dst, int64_t n, hipStream_t st) {
  if (n == 0) return hipSuccess;
  hipLaunchKernelGGL(to_bf16_kernel, dim3((unsigned)((n / 4 + 255) / 256)), dim3(256), 0, st,
                     src, (uint16_t*)dst, n);
  return hipGetLastError();
}

}  // namespace dash
