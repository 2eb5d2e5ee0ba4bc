// Staging of one 64-key block of K and V into LDS for the MFMA attention
// kernels (NTH threads per workgroup).
//
// K is stored row-major, Ks[key][d] with a 16-byte pad per row (row stride
// D + 8 elements): 16 lanes reading 16 consecutive rows at the same column
// then hit 16 distinct 4-bank groups.
//
// V is stored transposed, Vt[d][col] (row stride 72 elements), because the
// PV product contracts over keys and each MFMA operand lane needs 8 (or 4)
// consecutive keys of one dimension.  The column order is the order in which
// the score tiles hand their values to the PV MFMA: score tile t of a block
// holds keys 16t .. 16t+15, lane group g of its output holds keys
// 16t + 4g + j (j = 0..3), and a 32-key PV step s takes k-slots 8g .. 8g+7
// from tiles 2s (j) and 2s+1 (4 + j).  So key kappa = 32s + 16a + 4g + b
// sits in column 32s + 8g + 4a + b.
#pragma once

#include "dash_device.h"

namespace dash {

template <int D, int NTH>
struct StageCfg {
  static constexpr int KSTR = D + 8;           // Ks row stride (elements)
  static constexpr int VSTR = 72;              // Vt row stride (elements)
  static constexpr int TPR = D / 8;            // 16-byte pieces per key row
  static constexpr int KPT = (64 * TPR) / NTH; // rows per thread (1, 2 or 4)
  static constexpr int KS_ELEMS = 64 * KSTR;
  static constexpr int VT_ELEMS = D * VSTR;
  static_assert(KPT == 1 || KPT == 2 || KPT == 4, "staging split");
};

__device__ __forceinline__ int vt_col(int key) {
  return (key & ~31) | (((key >> 2) & 3) << 3) | (((key >> 4) & 1) << 2) | (key & 3);
}

// Global -> registers.  Keys key0 .. key0+63 of KV head h in a [*, Hkv, D]
// token-major tensor whose row 0 is `base_row`; keys at or past `kend` read 0.
template <int D, int NTH>
struct StageRegs {
  u32x4 k[StageCfg<D, NTH>::KPT];
  u32x4 v[StageCfg<D, NTH>::KPT];
};

template <int D, int NTH>
__device__ __forceinline__ void stage_load(StageRegs<D, NTH>& R, const uint16_t* __restrict__ kp,
                                           const uint16_t* __restrict__ vp, int64_t base_row,
                                           int key0, int kend, int Hkv, int h, int tid) {
  using C = StageCfg<D, NTH>;
  // K: thread -> (row kr + i * 256/TPR, piece)
  const int piece = tid % C::TPR;
  const int kr = tid / C::TPR;
#pragma unroll
  for (int i = 0; i < C::KPT; ++i) {
    const int key = key0 + kr + i * (NTH / C::TPR);
    u32x4 z = {0u, 0u, 0u, 0u};
    if (key < kend) z = ldg16(kp + ((base_row + key) * Hkv + h) * (int64_t)D + piece * 8);
    R.k[i] = z;
  }
  // V: thread -> (KPT consecutive keys, piece) so the transpose writes are
  // KPT-element runs of one dimension
  constexpr int NKG = 64 / C::KPT;  // key groups
  const int kg = tid % NKG;
  const int vpiece = tid / NKG;
#pragma unroll
  for (int i = 0; i < C::KPT; ++i) {
    const int key = key0 + kg * C::KPT + i;
    u32x4 z = {0u, 0u, 0u, 0u};
    if (key < kend) z = ldg16(vp + ((base_row + key) * Hkv + h) * (int64_t)D + vpiece * 8);
    R.v[i] = z;
  }
}

// Registers -> LDS.
template <int D, int NTH>
__device__ __forceinline__ void stage_store(const StageRegs<D, NTH>& R, uint16_t* Ks,
                                            uint16_t* Vt, int tid) {
  using C = StageCfg<D, NTH>;
  const int piece = tid % C::TPR;
  const int kr = tid / C::TPR;
#pragma unroll
  for (int i = 0; i < C::KPT; ++i) {
    const int row = kr + i * (NTH / C::TPR);
    *reinterpret_cast<u32x4*>(Ks + row * C::KSTR + piece * 8) = R.k[i];
  }
  constexpr int NKG = 64 / C::KPT;
  const int kg = tid % NKG;
  const int vpiece = tid / NKG;
  const int col0 = vt_col(kg * C::KPT);
  // element e of the 8 dims vpiece*8 + e; key i in register R.v[i]
#pragma unroll
  for (int e = 0; e < 8; ++e) {
    const int d = vpiece * 8 + e;
    const int w = e >> 1;
    const bool hi = e & 1;
    if constexpr (C::KPT == 4) {
      uint32_t x0 = hi ? (R.v[0][w] >> 16) : (R.v[0][w] & 0xffffu);
      uint32_t x1 = hi ? (R.v[1][w] >> 16) : (R.v[1][w] & 0xffffu);
      uint32_t x2 = hi ? (R.v[2][w] >> 16) : (R.v[2][w] & 0xffffu);
      uint32_t x3 = hi ? (R.v[3][w] >> 16) : (R.v[3][w] & 0xffffu);
      u32x2 pk = {x0 | (x1 << 16), x2 | (x3 << 16)};
      *reinterpret_cast<u32x2*>(Vt + d * C::VSTR + col0) = pk;
    } else if constexpr (C::KPT == 2) {
      uint32_t x0 = hi ? (R.v[0][w] >> 16) : (R.v[0][w] & 0xffffu);
      uint32_t x1 = hi ? (R.v[1][w] >> 16) : (R.v[1][w] & 0xffffu);
      *reinterpret_cast<uint32_t*>(Vt + d * C::VSTR + col0) = x0 | (x1 << 16);
    } else {
      Vt[d * C::VSTR + col0] = (uint16_t)(hi ? (R.v[0][w] >> 16) : (R.v[0][w] & 0xffffu));
    }
  }
}

}  // namespace dash
