// Exact merge of two partial attention results of the same query rows over
// disjoint key sets: the combine step of attention split along the keys
// across devices (ring attention), where each device attends its queries to
// one shard of K/V at a time and keeps a running (O, LSE).
//
// With LSE = m + ln l and O = acc / l for each part, the parts' states
// (m, l, acc) merge exactly after rescaling to a common maximum ("Ch. 3: MHA
// Limitations, MQA, GQA, and FlashAttention", 3.5; the rescale step of the
// online softmax): M = max(LSE_a, LSE_b), w = exp(LSE - M),
// O = (w_a O_a + w_b O_b) / (w_a + w_b), LSE = M + ln(w_a + w_b).
//
// HBM-bound elementwise pass: each thread moves 16 bytes of O (8 bf16
// features) of one (row, head) at a time, two such pieces per loop trip; the
// lanes of a row sit in one wave, so an in-place merge (out = o_a,
// lse_out = lse_a) reads every value before any lane of that row writes.
#include "device_common.h"
#include "launch.h"
#include "merge.h"

namespace attn {
namespace {

struct MergeParams {
  const uint16_t* oa;
  const float* la;
  const uint16_t* ob;
  const float* lb;
  uint16_t* o;
  float* lse;
  int B, N, H;
  long long rows;  // B * N * H (row, head) pairs
};

// ca * xa + cb * xb with both products rounded to float before the add.
__device__ __forceinline__ float sym_sum(float ca, float xa, float cb, float xb) {
#pragma clang fp contract(off)
  return ca * xa + cb * xb;
}

// One (row, head) piece: the lane's 16 bytes of O from each side and the
// row's two LSE values, loaded before any arithmetic.
struct Piece {
  u32x4 xa, xb;
  float la, lb;
};

template <int D, typename I>
__device__ __forceinline__ void piece_index(const MergeParams& p, I t, I& r, I& li) {
  constexpr int LPR = D / 8;
  r = t / LPR;  // (b * N + i) * H + h
  const I h = r % p.H;
  const I bi = r / p.H;
  const I i = bi % p.N;
  const I b = bi / p.N;
  li = (b * p.H + h) * p.N + i;  // [B, H, N]
}

template <int D, typename I>
__device__ __forceinline__ Piece load_piece(const MergeParams& p, I r, I li, int sub) {
  Piece x;
  x.la = p.la[li];
  x.lb = p.lb[li];
  // O is read once (non-temporal); the LSE lines serve the neighbouring rows
  x.xa = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(p.oa + (int64_t)r * D + sub * 8));
  x.xb = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(p.ob + (int64_t)r * D + sub * 8));
  return x;
}

template <int D, typename I>
__device__ __forceinline__ void merge_piece(const MergeParams& p, const Piece& x, I r, I li, int sub) {
  const bool nan = x.la != x.la || x.lb != x.lb;
  const float m = fmaxf(x.la, x.lb);
  float wa = 0.f, wb = 0.f;
  if (m != kNegInf) {
    wa = fast_exp2((x.la - m) * kLog2e);
    wb = fast_exp2((x.lb - m) * kLog2e);
  }
  const float sum = wa + wb;
  const float inv = nan ? __builtin_nanf("") : sum > 0.f ? 1.f / sum : 0.f;
  const float ca = wa * inv, cb = wb * inv;
  // Each product is rounded on its own and then added (no contraction into
  // an FMA, whose single rounding would depend on which side is the addend),
  // so merge(a, b) and merge(b, a) agree bit for bit.
  u32x4 y;
#pragma unroll
  for (int j = 0; j < 4; ++j)
    y[j] = pack_bf16x2(sym_sum(ca, bf16lo_to_f32(x.xa[j]), cb, bf16lo_to_f32(x.xb[j])),
                       sym_sum(ca, bf16hi_to_f32(x.xa[j]), cb, bf16hi_to_f32(x.xb[j])));
  *reinterpret_cast<u32x4*>(p.o + (int64_t)r * D + sub * 8) = y;
  if (sub == 0 && p.lse != nullptr)
    p.lse[li] = nan ? __builtin_nanf("") : sum > 0.f ? m + fast_log2(sum) * kLn2 : kNegInf;
}

// Two pieces per thread and trip (t and t + stride), both loaded before
// either is merged, so that each wave keeps twice the bytes in flight.  I is
// the index type: 32-bit when the piece count fits, 64-bit otherwise.  A
// piece's lanes stay in one wave (stride is a multiple of 256), so an
// in-place merge still reads a row's values before any lane writes them.
template <int D, typename I>
__global__ __launch_bounds__(256) void merge_kernel(const MergeParams p) {
  constexpr int LPR = D / 8;  // lanes per (row, head): 16 bytes each
  static_assert(64 % LPR == 0, "a (row, head) stays within one wave");
  const int sub = threadIdx.x % LPR;
  const I total = (I)p.rows * LPR;
  const I stride = (I)gridDim.x * 256;
  for (I t = (I)blockIdx.x * 256 + threadIdx.x; t < total; t += 2 * stride) {
    const I t2 = t + stride;
    const bool two = t2 < total;
    I r, li, r2, li2;
    piece_index<D, I>(p, t, r, li);
    piece_index<D, I>(p, two ? t2 : t, r2, li2);
    const Piece x = load_piece<D, I>(p, r, li, sub);
    const Piece x2 = load_piece<D, I>(p, r2, li2, sub);
    merge_piece<D, I>(p, x, r, li, sub);
    if (two) merge_piece<D, I>(p, x2, r2, li2, sub);
  }
}

}  // namespace

hipError_t launch_merge(const MergeArgs& a, hipStream_t stream) {
  MergeParams p;
  p.oa = static_cast<const uint16_t*>(a.o_a);
  p.la = a.lse_a;
  p.ob = static_cast<const uint16_t*>(a.o_b);
  p.lb = a.lse_b;
  p.o = static_cast<uint16_t*>(a.out);
  p.lse = a.lse_out;
  p.B = a.B;
  p.N = a.N;
  p.H = a.H;
  p.rows = (long long)a.B * a.N * a.H;
  if (p.rows == 0) return hipSuccess;
  const long long threads = p.rows * (a.d / 8);
  const long long blocks = (threads + 255) / 256;
  const int cap = device_cus() * 8;  // a grid-stride loop beyond this
  const dim3 grid((unsigned)(blocks < cap ? blocks : cap));
  // 32-bit indices while every piece index, and the index one grid past the
  // last, stays below 2^31
  const bool narrow = threads + 2LL * grid.x * 256 < (1LL << 31);
  if (a.d == 128) {
    if (narrow)
      hipLaunchKernelGGL((merge_kernel<128, int>), grid, dim3(256), 0, stream, p);
    else
      hipLaunchKernelGGL((merge_kernel<128, long long>), grid, dim3(256), 0, stream, p);
  } else {
    if (narrow)
      hipLaunchKernelGGL((merge_kernel<64, int>), grid, dim3(256), 0, stream, p);
    else
      hipLaunchKernelGGL((merge_kernel<64, long long>), grid, dim3(256), 0, stream, p);
  }
  return hipGetLastError();
}

}  // namespace attn
