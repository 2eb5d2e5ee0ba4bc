// Device helpers shared by the DashAttention HIP kernels (gfx950, wave64).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include <type_traits>

namespace dash {

constexpr int kWave = 64;
constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef short s16x4 __attribute__((ext_vector_type(4)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

// f(integral_constant<int, I>) for I = B .. E-1, unrolled at compile time.
template <int B, int E, typename F>
__device__ __forceinline__ void static_for(F&& f) {
  if constexpr (B < E) {
    f(std::integral_constant<int, B>());
    static_for<B + 1, E>(f);
  }
}

// ---------------------------------------------------------------- bf16

__device__ __forceinline__ float bf16_to_f32(uint32_t b) {
  return __uint_as_float(b << 16);
}
__device__ __forceinline__ float bf16lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf16hi(uint32_t w) { return __uint_as_float(w & 0xffff0000u); }

// fp32 -> bf16, round to nearest, ties to even (inputs are finite).
__device__ __forceinline__ uint32_t f32_to_bf16(float f) {
  uint32_t u = __float_as_uint(f);
  u += 0x7fffu + ((u >> 16) & 1u);
  return u >> 16;
}
__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
  return f32_to_bf16(lo) | (f32_to_bf16(hi) << 16);
}

// ---------------------------------------------------------------- wave reductions

__device__ __forceinline__ float wave_sum(float v) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) v += __shfl_xor(v, o);
  return v;
}
__device__ __forceinline__ float wave_max(float v) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) v = fmaxf(v, __shfl_xor(v, o));
  return v;
}
__device__ __forceinline__ float wave_min(float v) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) v = fminf(v, __shfl_xor(v, o));
  return v;
}
__device__ __forceinline__ int wave_sum_i(int v) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) v += __shfl_xor(v, o);
  return v;
}

// Reductions over the 16 lanes of a DPP row (lanes 16r .. 16r+15), every lane
// of the row receiving the result: quad xor 1, quad xor 2, half-row mirror
// (lane i <-> 7-i), row mirror (lane i <-> 15-i).
template <int CTRL>
__device__ __forceinline__ float dpp_f(float v) {
  return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), CTRL, 0xF, 0xF, false));
}
constexpr int kDppQuadXor1 = 0xB1;   // quad_perm [1,0,3,2]
constexpr int kDppQuadXor2 = 0x4E;   // quad_perm [2,3,0,1]
constexpr int kDppRowMirror = 0x140;
constexpr int kDppRowHalfMirror = 0x141;

__device__ __forceinline__ float row16_sum(float v) {
  v += dpp_f<kDppQuadXor1>(v);
  v += dpp_f<kDppQuadXor2>(v);
  v += dpp_f<kDppRowHalfMirror>(v);
  v += dpp_f<kDppRowMirror>(v);
  return v;
}
__device__ __forceinline__ float row16_max(float v) {
  v = fmaxf(v, dpp_f<kDppQuadXor1>(v));
  v = fmaxf(v, dpp_f<kDppQuadXor2>(v));
  v = fmaxf(v, dpp_f<kDppRowHalfMirror>(v));
  v = fmaxf(v, dpp_f<kDppRowMirror>(v));
  return v;
}
__device__ __forceinline__ float row16_min(float v) {
  v = fminf(v, dpp_f<kDppQuadXor1>(v));
  v = fminf(v, dpp_f<kDppQuadXor2>(v));
  v = fminf(v, dpp_f<kDppRowHalfMirror>(v));
  v = fminf(v, dpp_f<kDppRowMirror>(v));
  return v;
}

// Cross-row exchanges on gfx950 without LDS: value of lane l ^ 32 and l ^ 16.
__device__ __forceinline__ float xor32(float v) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(v), __float_as_uint(v), false,
                                                  false);
  // lanes < 32 get the upper half in r[1]; lanes >= 32 get the lower half in r[0]
  return __uint_as_float((threadIdx.x & 32) ? r[0] : r[1]);
}
__device__ __forceinline__ float xor16(float v) {
  const auto r = __builtin_amdgcn_permlane16_swap(__float_as_uint(v), __float_as_uint(v), false,
                                                  false);
  return __uint_as_float((threadIdx.x & 16) ? r[0] : r[1]);
}

// A 64-bit value every lane holds the same copy of, moved to scalar registers.
__device__ __forceinline__ int64_t uniform64(int64_t v) {
  const int lo = __builtin_amdgcn_readfirstlane((int)(uint32_t)v);
  const int hi = __builtin_amdgcn_readfirstlane((int)(v >> 32));
  return (int64_t)(((uint64_t)(uint32_t)hi << 32) | (uint32_t)lo);
}

// Two fp32 -> packed bf16x2 (round to nearest even, hardware conversion).
typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
typedef float f32x2_t __attribute__((ext_vector_type(2)));
// c + lo + hi of a packed bf16 pair, in fp32 (v_dot2 against (1, 1)).
__device__ __forceinline__ float dot2_bf16_ones(uint32_t pk, float c) {
  typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
  return __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2_t, pk),
                                         __builtin_bit_cast(bf16x2_t, 0x3f803f80u), c, false);
}

__device__ __forceinline__ uint32_t cvt_pk_bf16(float lo, float hi) {
  const f32x2_t v = {lo, hi};
  return __builtin_bit_cast(uint32_t, __builtin_convertvector(v, bf16x2_t));
}

// ---------------------------------------------------------------- sequences

// Where a sequence lives in the packed token and summary arrays.
struct SeqInfo {
  int64_t start;      // first token row
  int32_t len;        // tokens
  int64_t chunk_off;  // first summary row
};

// cu_seqlens == nullptr: fixed-length batch of max_seqlen tokens each.
// cu_chunks may be null for callers that do not use chunk_off.
__device__ __forceinline__ SeqInfo seq_info(const int32_t* cu_seqlens,
                                            const int32_t* cu_chunks, int s,
                                            int max_seqlen, int B) {
  SeqInfo r;
  if (cu_seqlens) {
    int a = cu_seqlens[s];
    r.start = a;
    r.len = cu_seqlens[s + 1] - a;
    r.chunk_off = cu_chunks ? cu_chunks[s] : 0;
  } else {
    r.start = (int64_t)s * max_seqlen;
    r.len = max_seqlen;
    r.chunk_off = (int64_t)s * (max_seqlen / B);
  }
  return r;
}

// Largest s with cu_seqlens[s] <= t (t a valid packed token row).
__device__ __forceinline__ int find_seq(const int32_t* cu_seqlens, int num_seqs,
                                        int64_t t) {
  int lo = 0, hi = num_seqs - 1;
  while (lo < hi) {
    int mid = (lo + hi + 1) >> 1;
    if ((int64_t)cu_seqlens[mid] <= t) lo = mid; else hi = mid - 1;
  }
  return lo;
}

// Bits of mask word w that name chunks c < n.
__device__ __forceinline__ unsigned long long routable_bits(int w, int n) {
  const int k = n - 64 * w;
  if (k <= 0) return 0ull;
  if (k >= 64) return ~0ull;
  return (1ull << k) - 1ull;
}

// ---------------------------------------------------------------- memory

__device__ __forceinline__ u32x4 ldg16(const void* p) {
  return *reinterpret_cast<const u32x4*>(p);
}

__device__ __forceinline__ bf16x8 as_bf16x8(u32x4 v) {
  return __builtin_bit_cast(bf16x8, v);
}
__device__ __forceinline__ s16x4 as_s16x4(u32x2 v) {
  return __builtin_bit_cast(s16x4, v);
}

// D(16x16, fp32) += A(16x32, bf16) * B(32x16, bf16).  Lane l supplies
// A[l%16][8(l/16)..+7] and B[8(l/16)..+7][l%16]; it receives D[4(l/16)+j][l%16].
__device__ __forceinline__ f32x4 mfma16x16x32(bf16x8 a, bf16x8 b, f32x4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
}
// D(16x16, fp32) += A(16x16, bf16) * B(16x16, bf16).  Lane l supplies
// A[l%16][4(l/16)..+3] and B[4(l/16)..+3][l%16].
__device__ __forceinline__ f32x4 mfma16x16x16(s16x4 a, s16x4 b, f32x4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(a, b, c, 0, 0, 0);
}

// (the asm below sets M0 on purpose: its clobber is declared)
#pragma clang diagnostic push
#pragma clang diagnostic ignored "-Winline-asm"
// Direct global->LDS loads, issued from asm so that the compiler neither
// tracks nor waits on them: the data lands in LDS, no register is written,
// the address registers are consumed at issue, and the ring's own counted
// vmcnt waits plus a barrier order them before every read.  (Vector-memory
// operations the compiler does not know about can only make its own counted
// waits stricter.)
//   lds_dma16: lane l writes LDS bytes lds_base + 16 l .. +15
//   lds_dma4 : lane l writes LDS bytes lds_base + 4 l .. +3
// (lds_base wave-uniform; lanes outside exec write nothing).
__device__ __forceinline__ void lds_dma16(const void* gptr, uint32_t lds_base) {
  asm volatile("s_mov_b32 m0, %0\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %1, off"
               :
               : "s"(lds_base), "v"(gptr)
               : "memory", "m0");
}
__device__ __forceinline__ void lds_dma4(const void* gptr, uint32_t lds_base) {
  asm volatile("s_mov_b32 m0, %0\n\ts_nop 0\n\tglobal_load_lds_dword %1, off"
               :
               : "s"(lds_base), "v"(gptr)
               : "memory", "m0");
}

// The same with a wave-uniform 64-bit base (SGPRs) and a 32-bit per-lane byte
// offset: address = sbase + voff.
__device__ __forceinline__ void lds_dma16s(const void* sbase, uint32_t voff, uint32_t lds_base) {
  asm volatile("s_mov_b32 m0, %0\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %1, %2"
               :
               : "s"(lds_base), "v"(voff), "s"(sbase)
               : "memory", "m0");
}
#pragma clang diagnostic pop

// LDS byte offset of a __shared__ object (a compile-time constant for the
// ring's static arrays).
__device__ __forceinline__ uint32_t lds_addr(const void* p) {
  return (uint32_t)(uintptr_t)(const __attribute__((address_space(3))) void*)p;
}

// LDS pointers proper (address space 3): offsets added to them fold into the
// reads' offset field.
typedef const __attribute__((address_space(3))) uint8_t lds_u8;
__device__ __forceinline__ u32x4 lds_read16(lds_u8* p) {
  typedef const __attribute__((address_space(3))) u32x4 lds_u32x4;
  return *reinterpret_cast<lds_u32x4*>(p);
}

// Transposing LDS read of 16-bit elements, 8 bytes a lane (gfx950): within
// each group of 16 lanes, lane i receives as its element j element i % 4 of
// the 8 bytes that lane 4 j + i / 4 of the group points at.  With lane a
// pointing at 4 consecutive columns 4 (a % 4) .. +3 of row a / 4 of a
// row-major tile, lane i thus receives column i of rows 0..3: the operand
// layout of a 16x16x16 MFMA for the tile's transpose.
__device__ __forceinline__ s16x4 lds_read_tr8(lds_u8* p) {
  typedef __attribute__((address_space(3))) s16x4 lds_s16x4;
  return __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4*)p);
}

// Slot of 16-byte piece pc of row j of a staged tile of D-dim bf16 rows
// (query heads of one token, or keys): pc ^ head_row_swz(j), which gives
// the rows that share the 64 banks (one 256-byte row at D = 128, two
// 128-byte rows at D = 64) distinct even offsets.  Then eight consecutive
// rows' 16-byte reads of one piece (an MFMA operand with the dims as k) and
// four consecutive rows' 8-byte transposing reads of two adjacent pieces (an
// operand with the rows as k) each touch every bank at most once.
template <int D>
__device__ __forceinline__ int head_row_swz(int j) {
  return D == 128 ? (2 * j) & 15 : j & 6;
}

// s_waitcnt for at most N outstanding vector-memory operations (N < 64) and
// no outstanding LDS operation
template <int N>
__device__ __forceinline__ void wait_vm() {
  static_assert(N >= 0 && N < 64, "vmcnt range");
  __builtin_amdgcn_s_waitcnt((N & 15) | ((N >> 4) << 14) | (7 << 4));
}

}  // namespace dash
