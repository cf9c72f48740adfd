// Device-side helpers shared by the gfx950 attention kernels.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace attn {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;
constexpr float kNegInf = -__builtin_inff();

// bf16 <-> f32.  bf16 is the high half of an f32; conversion to bf16 is the
// hardware round-to-nearest-even pack (v_cvt_pk_bf16_f32 on gfx950).
__device__ __forceinline__ float bf16lo_to_f32(uint32_t packed) {
  return __builtin_bit_cast(float, packed << 16);
}
__device__ __forceinline__ float bf16hi_to_f32(uint32_t packed) {
  return __builtin_bit_cast(float, packed & 0xffff0000u);
}
__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
  bf16x2 v;
  v[0] = (__bf16)lo;
  v[1] = (__bf16)hi;
  return __builtin_bit_cast(uint32_t, v);
}

// Reinterpret a packed bf16 pair.  Always pass the word by value: clang
// mis-compiles __builtin_bit_cast applied directly to an ext-vector element
// (v[i]) and reads element 0 whatever the index.
__device__ __forceinline__ bf16x2 as_bf16x2(uint32_t u) { return __builtin_bit_cast(bf16x2, u); }

__device__ __forceinline__ float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }
__device__ __forceinline__ float fast_log2(float x) { return __builtin_amdgcn_logf(x); }

// Work-group id remap so that consecutive logical work items land on the
// same XCD.  Work groups are handed to the 8 XCDs round-robin by id, so
// physical id i runs on XCD i % 8; logical items [x*per + min(x,rem), ...)
// are given to XCD x.  The map is a bijection on [0, total).
__device__ __forceinline__ int xcd_remap(int pid, int total) {
  constexpr int kXcd = 8;
  const int per = total / kXcd;
  const int rem = total % kXcd;
  const int x = pid % kXcd;
  const int k = pid / kXcd;
  return x * per + (x < rem ? x : rem) + k;
}

// Cross-lane helpers (wave64).
__device__ __forceinline__ float swap_halves(float x) {
  // value held by lane (l ^ 32)
  return __shfl_xor(x, 32, 64);
}

template <int CTRL>
__device__ __forceinline__ float dpp_f32(float x) {
  return __builtin_bit_cast(
      float, __builtin_amdgcn_mov_dpp(__builtin_bit_cast(int, x), CTRL, 0xF, 0xF, false));
}
// DPP controls: quad_perm [1,0,3,2] (lane ^ 1), [2,3,0,1] (lane ^ 2),
// row_half_mirror (lane i <-> 7 - i within each 8), row_ror:8 (lane ^ 8 within 16)
constexpr int kDppXor1 = 0xB1;
constexpr int kDppXor2 = 0x4E;
constexpr int kDppHalfMirror = 0x141;
constexpr int kDppRor8 = 0x128;

__device__ __forceinline__ int clampi(int x, int lo, int hi) { return min(max(x, lo), hi); }

// Packed sequences: the sequence whose schedule slots hold slot v, i.e. the
// largest s in [0, n) with start(s) = cu[s] / TILE + s <= v (start is strictly
// increasing for nondecreasing cu; cu is clamped to [0, total] as read).  A
// 64-way search: each round the wave's lanes test 64 evenly spaced
// candidates and the count of passing lanes narrows the range 64-fold.  The
// result stays in [0, n) whatever cu holds.  A sequence's TILE-row tiles
// fit in its slots: start(s + 1) - start(s) >= ceil(len(s) / TILE).
// cu may point to global memory or to LDS (Ptr: a pointer to const int in
// either address space).
template <int TILE, typename Ptr>
__device__ __forceinline__ int find_seq(Ptr cu, int n, int total, int v, int lane) {
  int lo = 0, hi = n;
  while (hi - lo > 1) {
    const int step = (hi - lo + 63) / 64;
    const int idx = lo + lane * step;
    bool pass = false;
    if (idx < hi) pass = clampi(cu[idx], 0, total) / TILE + idx <= v;
    const int cnt = __builtin_popcountll(__builtin_amdgcn_ballot_w64(pass));
    lo += (max(cnt, 1) - 1) * step;
    hi = min(hi, lo + step);
  }
  return __builtin_amdgcn_readfirstlane(lo);
}

}  // namespace attn
