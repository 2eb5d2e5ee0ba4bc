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

// Global -> registers with this thread's addresses computed once: K row
// kr + i*NTH/TPR, piece `piece`; V rows kg*KPT + i, piece `vpiece`.  load()
// reads a block that lies inside the sequence; load_guarded() reads 0 for keys
// at or past kend.
template <int D, int NTH>
struct Stager {
  using C = StageCfg<D, NTH>;
  static constexpr int NKG = 64 / C::KPT;
  const uint16_t* kptr;
  const uint16_t* vptr;
  int64_t rowstride;  // elements between consecutive tokens (Hkv * D)
  int kr, kg;
  __device__ __forceinline__ Stager(const uint16_t* kp, const uint16_t* vp, int64_t base_row,
                                    int Hkv, int h, int tid) {
    const int piece = tid % C::TPR;
    kr = tid / C::TPR;
    kg = tid % NKG;
    const int vpiece = tid / NKG;
    rowstride = (int64_t)Hkv * D;
    kptr = kp + (base_row + kr) * rowstride + (int64_t)h * D + piece * 8;
    vptr = vp + (base_row + kg * C::KPT) * rowstride + (int64_t)h * D + vpiece * 8;
  }
  __device__ __forceinline__ void load(StageRegs<D, NTH>& R, int key0) const {
    const uint16_t* kb = kptr + key0 * rowstride;
    const uint16_t* vb = vptr + key0 * rowstride;
#pragma unroll
    for (int i = 0; i < C::KPT; ++i) R.k[i] = ldg16(kb + i * (NTH / C::TPR) * rowstride);
#pragma unroll
    for (int i = 0; i < C::KPT; ++i) R.v[i] = ldg16(vb + i * rowstride);
  }
  __device__ __forceinline__ void load_guarded(StageRegs<D, NTH>& R, int key0, int kend) const {
    const uint16_t* kb = kptr + key0 * rowstride;
    const uint16_t* vb = vptr + key0 * rowstride;
#pragma unroll
    for (int i = 0; i < C::KPT; ++i) {
      u32x4 z = {0u, 0u, 0u, 0u};
      if (key0 + kr + i * (NTH / C::TPR) < kend) z = ldg16(kb + i * (NTH / C::TPR) * rowstride);
      R.k[i] = z;
    }
#pragma unroll
    for (int i = 0; i < C::KPT; ++i) {
      u32x4 z = {0u, 0u, 0u, 0u};
      if (key0 + kg * C::KPT + i < kend) z = ldg16(vb + i * rowstride);
      R.v[i] = z;
    }
  }
};

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
  // dims vpiece*8 + 2w (low halves) and + 2w + 1 (high halves) of the KPT keys
#pragma unroll
  for (int w = 0; w < 4; ++w) {
    const int d = vpiece * 8 + 2 * w;
    if constexpr (C::KPT == 4) {
      const u32x2 lo = {__builtin_amdgcn_perm(R.v[1][w], R.v[0][w], 0x05040100u),
                        __builtin_amdgcn_perm(R.v[3][w], R.v[2][w], 0x05040100u)};
      const u32x2 hi = {__builtin_amdgcn_perm(R.v[1][w], R.v[0][w], 0x07060302u),
                        __builtin_amdgcn_perm(R.v[3][w], R.v[2][w], 0x07060302u)};
      *reinterpret_cast<u32x2*>(Vt + d * C::VSTR + col0) = lo;
      *reinterpret_cast<u32x2*>(Vt + (d + 1) * C::VSTR + col0) = hi;
    } else if constexpr (C::KPT == 2) {
      *reinterpret_cast<uint32_t*>(Vt + d * C::VSTR + col0) =
          __builtin_amdgcn_perm(R.v[1][w], R.v[0][w], 0x05040100u);
      *reinterpret_cast<uint32_t*>(Vt + (d + 1) * C::VSTR + col0) =
          __builtin_amdgcn_perm(R.v[1][w], R.v[0][w], 0x07060302u);
    } else {
      Vt[d * C::VSTR + col0] = (uint16_t)(R.v[0][w] & 0xffffu);
      Vt[(d + 1) * C::VSTR + col0] = (uint16_t)(R.v[0][w] >> 16);
    }
  }
}

}  // namespace dash
