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
// bwd_dkdv_kernel: one workgroup of 4 waves per (64-key block, sequence, KV
// head); wave w owns keys 16w .. 16w+15 of the block and holds their K and V
// rows as MFMA operands for the whole kernel.  It scans the sequence's mask
// 256 rows at a time, compacts the rows that see the block (ballots and a
// block-wide prefix, in row order, so the sums are deterministic), and for
// each such row stages q_i, dO_i and their transposes in LDS:
//   S  = Q_i K_w^T and dP = dO_i V_w^T   (16 heads x 16 keys, 16x16x32 MFMA;
//                                         the accumulators of S are exactly
//                                         the operand layout P needs below)
//   P  = exp2(s S + b - LSE),  dS = P (dP - D)
//   dV_w^T += dO_i^T P,  dK_w^T += Q_i^T dS   (16x16x16 MFMA over the heads)
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

constexpr int kBkThreads = 256;

template <int D, int HT>
__global__ __launch_bounds__(kBkThreads) void bwd_dkdv_kernel(Geom g, BwdParams p, float* dk,
                                                              float* dv) {
  constexpr int G = 16 * HT;
  constexpr int KS = D / 32;
  constexpr int DT = D / 16;
  constexpr int NTH = kBkThreads;
  constexpr int QROW = D + 8;   // LDS row stride (elements) of Q / dO: [head][d]
  constexpr int TROW = G + 4;   // LDS row stride (elements) of Q^T / dO^T: [d][head]
  __shared__ __attribute__((aligned(16))) uint16_t Qs[G * QROW];
  __shared__ __attribute__((aligned(16))) uint16_t Ds[G * QROW];
  __shared__ __attribute__((aligned(16))) uint16_t Qt[D * TROW];
  __shared__ __attribute__((aligned(16))) uint16_t Dt[D * TROW];
  __shared__ float Ls[G], Dl[G];
  __shared__ float Bias;
  __shared__ int Rows[NTH];
  __shared__ int Wcnt[NTH / 64];

  const int tid = threadIdx.x, lane = tid & 63, wv = tid >> 6;
  const int r = lane & 15, gq = lane >> 4;
  const int blk = blockIdx.x, s = blockIdx.y, h = blockIdx.z;
  const SeqInfo si = seq_info(g.cu_seqlens, nullptr, s, g.max_seqlen, g.B);
  const int key0 = blk * 64;
  if (key0 >= si.len) return;
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
  f32x4 adk[DT], adv[DT];
#pragma unroll
  for (int dt = 0; dt < DT; ++dt) {
    adk[dt] = f32x4{0.f, 0.f, 0.f, 0.f};
    adv[dt] = f32x4{0.f, 0.f, 0.f, 0.f};
  }
  const float sl2 = p.scale * kLog2e;
  const int first = key0;  // rows before the block see none of its keys

  // staging of one row: registers (fetch, one row ahead) -> LDS (put)
  constexpr int NPC = (G * D / 8 + NTH - 1) / NTH;  // 16-byte pieces per thread
  u32x4 ra[NPC], rb[NPC];
  float rl = 0.f, rd = 0.f, rbias = 0.f;
  auto fetch = [&](int row) {
    const int64_t tok = si.start + row;
#pragma unroll
    for (int n = 0; n < NPC; ++n) {
      const int pc = tid + NTH * n;
      if (pc < G * D / 8) {
        const int hh = pc / (D / 8), d0 = (pc % (D / 8)) * 8;
        const int64_t src = (tok * g.Hq + h * G + hh) * (int64_t)D + d0;
        ra[n] = ldg16((const uint16_t*)p.q + src);
        rb[n] = ldg16((const uint16_t*)p.dout + src);
      }
    }
    if (tid < G) {
      const int64_t hr = (int64_t)(h * G + tid) * T + tok;
      rl = p.lse[hr] * kLog2e;
      rd = p.delta[hr];
    }
    if (tid == 0)
      rbias = row < cend ? 0.f : p.log_prior[((int64_t)h * T + tok) * g.C_slots + c] * kLog2e;
  };
  auto put = [&](int) {
#pragma unroll
    for (int n = 0; n < NPC; ++n) {
      const int pc = tid + NTH * n;
      if (pc < G * D / 8) {
        const int hh = pc / (D / 8), d0 = (pc % (D / 8)) * 8;
        const u32x4 a = ra[n], b = rb[n];
        *reinterpret_cast<u32x4*>(&Qs[hh * QROW + d0]) = a;
        *reinterpret_cast<u32x4*>(&Ds[hh * QROW + d0]) = b;
#pragma unroll
        for (int w = 0; w < 4; ++w) {
          Qt[(d0 + 2 * w) * TROW + hh] = (uint16_t)(a[w] & 0xFFFFu);
          Qt[(d0 + 2 * w + 1) * TROW + hh] = (uint16_t)(a[w] >> 16);
          Dt[(d0 + 2 * w) * TROW + hh] = (uint16_t)(b[w] & 0xFFFFu);
          Dt[(d0 + 2 * w + 1) * TROW + hh] = (uint16_t)(b[w] >> 16);
        }
      }
    }
    if (tid < G) {
      Ls[tid] = rl;
      Dl[tid] = rd;
    }
    if (tid == 0) Bias = rbias;
  };

  for (int r0 = first; r0 < si.len; r0 += NTH) {
    // ---- rows r0 .. r0+255 that see the block, compacted in order
    const int i = r0 + tid;
    bool on = false;
    if (i < si.len) {
      if (i < cend) {
        on = true;  // the block's own chunk: causal (i >= key0 here)
      } else {
        const unsigned long long w = mask[((int64_t)h * T + si.start + i) * g.W + (c >> 6)];
        on = (w >> (c & 63)) & 1ull;
      }
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
      const int row = Rows[k];
      if (k == 0) fetch(row);
      put(row);
      __syncthreads();
      if (k + 1 < total) fetch(Rows[k + 1]);  // in flight while this row computes
      const float bz = Bias;
      const bool masked = row < cend;  // the block's own chunk: keys after the row are unseen
#pragma unroll
      for (int ht = 0; ht < HT; ++ht) {
        f32x4 sacc = {0.f, 0.f, 0.f, 0.f}, pacc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int ks = 0; ks < KS; ++ks) {
          const u32x4 qa = *reinterpret_cast<const u32x4*>(&Qs[(16 * ht + r) * QROW + 32 * ks + 8 * gq]);
          const u32x4 da = *reinterpret_cast<const u32x4*>(&Ds[(16 * ht + r) * QROW + 32 * ks + 8 * gq]);
          sacc = mfma16x16x32(as_bf16x8(qa), kf[ks], sacc);
          pacc = mfma16x16x32(as_bf16x8(da), vf[ks], pacc);
        }
        // lane (gq, r): heads 16 ht + 4 gq + j, key mykey
        float pv[4], ds[4];
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          const int hh = 16 * ht + 4 * gq + j;
          float e = __builtin_amdgcn_exp2f(fmaf(sacc[j], sl2, bz - Ls[hh]));
          if (masked) e = mykey <= row ? e : 0.f;
          e = mykey <= kmax ? e : 0.f;
          pv[j] = e;
          ds[j] = e * (pacc[j] - Dl[hh]);
        }
        const u32x2 pb = {cvt_pk_bf16(pv[0], pv[1]), cvt_pk_bf16(pv[2], pv[3])};
        const u32x2 sb = {cvt_pk_bf16(ds[0], ds[1]), cvt_pk_bf16(ds[2], ds[3])};
#pragma unroll
        for (int dt = 0; dt < DT; ++dt) {
          // A = X^T tile: dims 16 dt + r, heads 16 ht + 4 gq .. +3
          const u32x2 ta = *reinterpret_cast<const u32x2*>(&Dt[(16 * dt + r) * TROW + 16 * ht + 4 * gq]);
          const u32x2 tq = *reinterpret_cast<const u32x2*>(&Qt[(16 * dt + r) * TROW + 16 * ht + 4 * gq]);
          adv[dt] = mfma16x16x16(as_s16x4(ta), as_s16x4(pb), adv[dt]);
          adk[dt] = mfma16x16x16(as_s16x4(tq), as_s16x4(sb), adk[dt]);
        }
      }
      __syncthreads();  // the staging buffers are refilled for the next row
    }
  }
  // ---- write this wave's keys: lane (gq, r) holds dims 16 dt + 4 gq .. +3 of key mykey
  if (mykey <= kmax) {
    const int64_t row = ((si.start + mykey) * g.Hkv + h) * (int64_t)D;
#pragma unroll
    for (int dt = 0; dt < DT; ++dt) {
      f32x4 wk = adk[dt];
#pragma unroll
      for (int j = 0; j < 4; ++j) wk[j] *= p.scale;
      *reinterpret_cast<f32x4*>(dk + row + 16 * dt + 4 * gq) = wk;
      *reinterpret_cast<f32x4*>(dv + row + 16 * dt + 4 * gq) = adv[dt];
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
  dim3 grid((g.max_seqlen + 63) / 64, g.num_seqs, g.Hkv);
#define DASH_BK(DD, HH)                                                                    \
  hipLaunchKernelGGL((bwd_dkdv_kernel<DD, HH>), grid, dim3(kBkThreads), 0, st, g, p, dk, dv)
  if (g.G == 16) {
    if (g.D == 64) DASH_BK(64, 1); else DASH_BK(128, 1);
  } else {
    if (g.D == 64) DASH_BK(64, 2); else DASH_BK(128, 2);
  }
#undef DASH_BK
  return hipGetLastError();
}

__global__ __launch_bounds__(256) void zero_kernel(float* __restrict__ x, int64_t n) {
  const int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (i < n) x[i] = 0.f;
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
