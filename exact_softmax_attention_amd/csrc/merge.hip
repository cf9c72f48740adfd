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
// features) of one (row, head); the lanes of a row sit in one wave, so an
// in-place merge (out = o_a, lse_out = lse_a) reads every value before any
// lane of that row writes.
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

template <int D>
__global__ __launch_bounds__(256) void merge_kernel(const MergeParams p) {
  constexpr int LPR = D / 8;  // lanes per (row, head): 16 bytes each
  static_assert(64 % LPR == 0, "a (row, head) stays within one wave");
  const int sub = threadIdx.x % LPR;
  for (long long t = (long long)blockIdx.x * 256 + threadIdx.x; t < p.rows * LPR;
       t += (long long)gridDim.x * 256) {
    const long long r = t / LPR;  // (b * N + i) * H + h
    const int h = (int)(r % p.H);
    const long long bi = r / p.H;
    const int i = (int)(bi % p.N);
    const long long b = bi / p.N;
    const long long li = (b * p.H + h) * p.N + i;  // [B, H, N]
    const float la = p.la[li], lb = p.lb[li];
    // O is read once (non-temporal); the LSE lines serve the neighbouring rows
    const u32x4 xa = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(p.oa + r * D + sub * 8));
    const u32x4 xb = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(p.ob + r * D + sub * 8));
    const bool nan = la != la || lb != lb;
    const float m = fmaxf(la, lb);
    float wa = 0.f, wb = 0.f;
    if (m != kNegInf) {
      wa = fast_exp2((la - m) * kLog2e);
      wb = fast_exp2((lb - m) * kLog2e);
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
      y[j] = pack_bf16x2(sym_sum(ca, bf16lo_to_f32(xa[j]), cb, bf16lo_to_f32(xb[j])),
                         sym_sum(ca, bf16hi_to_f32(xa[j]), cb, bf16hi_to_f32(xb[j])));
    *reinterpret_cast<u32x4*>(p.o + r * D + sub * 8) = y;
    if (sub == 0 && p.lse != nullptr)
      p.lse[li] = nan ? __builtin_nanf("") : sum > 0.f ? m + fast_log2(sum) * kLn2 : kNegInf;
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
  if (a.d == 128)
    hipLaunchKernelGGL(merge_kernel<128>, grid, dim3(256), 0, stream, p);
  else
    hipLaunchKernelGGL(merge_kernel<64>, grid, dim3(256), 0, stream, p);
  return hipGetLastError();
}

}  // namespace attn
