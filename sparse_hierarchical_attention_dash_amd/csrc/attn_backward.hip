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
// bwd_dkdv_kernel: one workgroup of 4 waves per (64-key block, slice of 4096
// rows, sequence, KV head); wave w owns keys 16w .. 16w+15 of the block and
// holds their K and V rows as MFMA operands for the whole kernel.  It scans
// its slice's mask words 1024 rows at a time, compacts the rows that see the
// block (ballots and a block-wide prefix, in row order), and streams those
// rows' q_i and dO_i through a ring of LDS stages filled by direct
// global->LDS loads (16-byte pieces XOR-swizzled per head, so that the
// operand reads below are free of bank conflicts; the row's LSE, D and bias
// beside them), several rows ahead of the one computed.  The transposed
// operands of the dV and dK products come from the same staged rows by
// gfx950's transposing LDS reads, so each row crosses the fabric once:
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

template <int D, int HT>
struct DkdvCfg {
  static constexpr int NW = 4;                         // waves: one 16-key tile each
  static constexpr int NTH = 64 * NW;
  static constexpr int G = 16 * HT;
  static constexpr int NS = 4;                         // ring stages, one row each
  static constexpr int ABYTES = G * D * 2;             // one array of one row
  static constexpr int SBYTES = 2 * ABYTES;            // Q, dO
  static constexpr int AU = ABYTES / 16;               // 16-byte units per array
  static constexpr int NUT = 2 * AU / NTH;             // unit loads per thread per stage
  static_assert(2 * AU % NTH == 0, "units per stage");
};

template <int D, int HT>
__global__ __launch_bounds__(256, HT == 1 ? 3 : 2) void bwd_dkdv_kernel(Geom g, BwdParams p, float* dk,
                                                       float* dv) {
  using C = DkdvCfg<D, HT>;
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

  // this wave's 16 keys: K and V rows as the B operand of Q K^T and dO V^T
  const int mykey = key0 + 16 * wv + r;
  bf16x8 kf[KS], vf[KS];
  {
    const int64_t row = ((si.start + min(mykey, kmax)) * g.Hkv + h) * (int64_t)D;
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) {
      kf[ks] = as_bf16x8(ldg16((const uint16_t*)p.k + row + 32 * ks + 8 * gq));
      vf[ks] = as_bf16x8(ldg16((const uint16_t*)p.v + row + 32 * ks + 8 * gq));
    }
  }
  // the operand loads complete here, so that the compiler's own waits for them
  // do not land inside the ring loop, where they would also wait for the ring
  wait_vm<0>();
  f32x4 adk[DT], adv[DT];
#pragma unroll
  for (int dt = 0; dt < DT; ++dt) {
    adk[dt] = f32x4{0.f, 0.f, 0.f, 0.f};
    adv[dt] = f32x4{0.f, 0.f, 0.f, 0.f};
  }
  const float sl2 = p.scale * kLog2e;
  // per-thread staging: piece e of this thread is 16 bytes of head j's row of
  // Q (or dO), at a fixed byte offset from the row's first head; a wave's
  // pieces lie all in Q or all in dO
  uint32_t poff[C::NUT];
  int parr[C::NUT];
#pragma unroll
  for (int e = 0; e < C::NUT; ++e) {
    const int U = tid + NTH * e;
    const int u = U % C::AU;
    // slot u % UPH of head j holds the piece head_row_swz places there
    const int j = u / UPH, pc = (u % UPH) ^ head_row_swz<D>(j);
    poff[e] = (uint32_t)((j * D + 8 * pc) * 2);
    parr[e] = __builtin_amdgcn_readfirstlane(U / C::AU);
  }
  // lanes < 2G: the LSE (lanes < G) or D of head lane % G, for token 0
  const float* scsrc = lane < G ? p.lse + (int64_t)(h * G + lane) * T + si.start
                                : p.delta + (int64_t)(h * G + (lane & (G - 1))) * T + si.start;
  const float* bzsrc = p.log_prior + ((int64_t)h * T + si.start) * g.C_slots + c;
  const int64_t qrs = (int64_t)g.Hq * D * 2;  // bytes between tokens of Q and dO

  // one row (wave-uniform) into ring slot `slot`: thread tid loads units
  // tid + 256 e
  auto issue = [&](int row, int slot) {
    const uint32_t base = lds_addr(Ring) + (uint32_t)(slot * C::SBYTES);
    const int64_t rb = (si.start + row) * qrs + (int64_t)h * G * D * 2;
#pragma unroll
    for (int e = 0; e < C::NUT; ++e)
      lds_dma16s((const uint8_t*)(parr[e] == 0 ? p.q : p.dout) + rb, poff[e],
                 __builtin_amdgcn_readfirstlane(base + (uint32_t)(16 * (NTH * e + 64 * wv))));
    if (lane < 2 * G)
      lds_dma4(scsrc + row, __builtin_amdgcn_readfirstlane(lds_addr(&Sc[slot][wv][0])));
    if (lane == 0)  // the bias (any valid word for rows of the block's own chunk)
      lds_dma4(bzsrc + (int64_t)row * g.C_slots,
               __builtin_amdgcn_readfirstlane(lds_addr(&Bz[slot][wv][0])));
  };

  // S and dP of one staged row and head tile, then P and dS packed as the B
  // operand's half: lane (gq, r) holds heads 16 ht + 4 gq + jj, key mykey.  A
  // row of the block's own chunk sees key j iff j <= row (row <= the
  // sequence's last key), with bias 0.
  auto row_terms = [&](int slot, int row, int ht, u32x2& pb, u32x2& sb) {
    const bool own = row < cend;
    lds_u8* Qs = (lds_u8*)(Ring + slot * C::SBYTES);
    lds_u8* Ds = Qs + C::ABYTES;
    const float bz = own ? 0.f : Bz[slot][wv][0] * kLog2e;
    f32x4 sacc = {0.f, 0.f, 0.f, 0.f}, pacc = {0.f, 0.f, 0.f, 0.f};
    const int j = 16 * ht + r;
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) {
      const int off = 16 * (j * UPH + ((4 * ks + gq) ^ head_row_swz<D>(j)));
      sacc = mfma16x16x32(as_bf16x8(lds_read16(Qs + off)), kf[ks], sacc);
      pacc = mfma16x16x32(as_bf16x8(lds_read16(Ds + off)), vf[ks], pacc);
    }
    float pv[4], ds[4];
#pragma unroll
    for (int jj = 0; jj < 4; ++jj) {
      const int hh = 16 * ht + 4 * gq + jj;
      float e = __builtin_amdgcn_exp2f(fmaf(sacc[jj], sl2, bz - Sc[slot][wv][hh] * kLog2e));
      if (own) e = mykey <= row ? e : 0.f;
      pv[jj] = e;
      ds[jj] = e * (pacc[jj] - Sc[slot][wv][G + hh]);
    }
    pb = u32x2{cvt_pk_bf16(pv[0], pv[1]), cvt_pk_bf16(pv[2], pv[3])};
    sb = u32x2{cvt_pk_bf16(ds[0], ds[1]), cvt_pk_bf16(ds[2], ds[3])};
  };
  // two staged rows per step (the second absent past the list's end): the
  // dV and dK products contract over (row, head), 32 at a time.  k-slot
  // 8 gq + 4 x + jj is head 16 ht + 4 gq + jj of row x; the transposing reads
  // (lane (gq, r) pointing at head 16 ht + 4 gq + r / 4, dims 16 dt + 4 (r % 4)
  // .. +3) give lane (gq, r) dim 16 dt + r of those heads.
  auto compute_pair = [&](int sa, int ra, int sbs, int rb) {
    const bool two = rb >= 0;
#pragma unroll
    for (int ht = 0; ht < HT; ++ht) {
      u32x2 pa, da, pbb = {0u, 0u}, dbb = {0u, 0u};
      row_terms(sa, ra, ht, pa, da);
      if (two) row_terms(sbs, rb, ht, pbb, dbb);
      const u32x4 pb4 = {pa[0], pa[1], pbb[0], pbb[1]};
      const u32x4 sb4 = {da[0], da[1], dbb[0], dbb[1]};
      lds_u8* Qa = (lds_u8*)(Ring + sa * C::SBYTES);
      lds_u8* Qb = (lds_u8*)(Ring + sbs * C::SBYTES);
      const int jt = 16 * ht + 4 * gq + (r >> 2);
      const int tbase = 16 * jt * UPH + 8 * (r & 1);
      const int tsw = head_row_swz<D>(jt), tpc = (r & 3) >> 1;
#pragma unroll
      for (int dt = 0; dt < DT; ++dt) {
        const int off = tbase + 16 * ((2 * dt + tpc) ^ tsw);
        const u32x2 ta0 = __builtin_bit_cast(u32x2, lds_read_tr8(Qa + C::ABYTES + off));
        const u32x2 tq0 = __builtin_bit_cast(u32x2, lds_read_tr8(Qa + off));
        u32x2 ta1 = {0u, 0u}, tq1 = {0u, 0u};
        if (two) {
          ta1 = __builtin_bit_cast(u32x2, lds_read_tr8(Qb + C::ABYTES + off));
          tq1 = __builtin_bit_cast(u32x2, lds_read_tr8(Qb + off));
        }
        const u32x4 ta = {ta0[0], ta0[1], ta1[0], ta1[1]};
        const u32x4 tq = {tq0[0], tq0[1], tq1[0], tq1[1]};
        adv[dt] = mfma16x16x32(as_bf16x8(ta), as_bf16x8(pb4), adv[dt]);
        adk[dt] = mfma16x16x32(as_bf16x8(tq), as_bf16x8(sb4), adk[dt]);
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

    // rows 2q and 2q + 1 in slots (2q) % 4 and (2q + 1) % 4: a step waits for
    // its two rows (the only loads in flight), and at its barrier every wave
    // has left the previous step's slots, which then take the next two rows
    issue(__builtin_amdgcn_readfirstlane(Rows[0]), 0);
    if (total > 1) issue(__builtin_amdgcn_readfirstlane(Rows[1]), 1);
    for (int k = 0; k < total; k += 2) {
      wait_vm<0>();
      __syncthreads();
#pragma unroll 1
      for (int n = k + 2; n < min(k + 4, total); ++n)
        issue(__builtin_amdgcn_readfirstlane(Rows[n]), n & 3);
      compute_pair(k & 3, __builtin_amdgcn_readfirstlane(Rows[k]), (k + 1) & 3,
                   k + 1 < total ? __builtin_amdgcn_readfirstlane(Rows[k + 1]) : -1);
    }
    __syncthreads();  // the ring and Rows are refilled
  }
  // ---- add this slice's sums for the wave's keys: lane (gq, r) holds dims
  // 16 dt + 4 gq .. +3 of key mykey
  if (seen > 0 && mykey <= kmax) {
    const int64_t row = ((si.start + mykey) * g.Hkv + h) * (int64_t)D;
#pragma unroll
    for (int dt = 0; dt < DT; ++dt) {
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        atomicAdd(dk + row + 16 * dt + 4 * gq + j, adk[dt][j] * p.scale);
        atomicAdd(dv + row + 16 * dt + 4 * gq + j, adv[dt][j]);
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
  hipLaunchKernelGGL((bwd_dkdv_kernel<DD, HH>), grid, dim3(DkdvCfg<DD, HH>::NTH), 0, st, g, p, \
                     dk, dv)
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
