// Single-query decode over a block-paged KV cache, split along the keys.
//
// Method: a decode step's one new query reads every cached K/V of its
// sequence ("Ch. 3: MHA Limitations, MQA, GQA, and FlashAttention", 3.1);
// the cache is split into fixed-size blocks reached through a lookup table
// ("Inference Engineering", 2.5); the keys are cut into splits whose partial
// softmax states (m, l, acc) are merged exactly afterwards (the rescale of
// "Ch. 3", 3.5: l e^m is invariant, so states rescaled to a common maximum
// add).
//
// Kernel 1 (split): one wave per (sequence, KV head, group of GH query heads,
// 256-token split).  Lane l = (token slot l / (D/8), feature slice l % (D/8)):
// each lane loads 8 features (16 contiguous bytes) of one token's K and V
// row, so a pass covers 64/(D/8) tokens and a 16-token block takes 4 passes
// (D = 128) or 2 (D = 64).  Scores: v_dot2_f32_bf16 on the bf16 pairs of q and
// k, then an all-reduce over the D/8 slices with DPP.
// Each lane keeps its own running max per head and only rescales when some
// lane's score exceeds its max by more than 2^8 (wave-uniform branch), which
// is exact algebra: the final merge divides by a sum taken at the same max.
// P V is accumulated in float32 on the lane's own feature slice.  At the end
// the token slots are merged (same rule) and one partial per query head is
// written to the workspace.  The next block's K/V loads are issued before the
// current block is computed; the small per-lane state lets two waves share a
// SIMD, which keeps enough loads in flight for the HBM bandwidth.
//
// Kernel 2 (combine): one work group per (sequence, query head); 4 waves each
// take every 4th split, rescale to the common maximum and sum in a fixed
// order; the 4 partial sums are added in LDS.  Deterministic: no atomics.
#include "device_common.h"
#include "launch.h"

namespace attn {
namespace {

constexpr int kBlock = 16;         // tokens per cache block
constexpr int kSplit = 256;        // tokens per split
constexpr int kSplitBlocks = kSplit / kBlock;
constexpr float kLazy = 8.0f;      // rescale only when a score passes max + 8 (base 2)
constexpr int kCombineWaves = 4;

struct Params {
  const uint16_t* q;
  const uint16_t* kc;
  const uint16_t* vc;
  const int* table;
  const int* lens;
  uint16_t* o;
  float* lse;
  float2* ws_ml;   // [B, Hq, max_splits] (m, l)
  float* ws_acc;   // [B, Hq, max_splits, D]
  int Hq, Hkv, group, hgroups, max_blocks, num_blocks, window, max_splits;
  float sl2;
};

__device__ __forceinline__ int split_lo_token(int L, int window) {
  return window > 0 ? max(0, L - window) : 0;
}

template <int GH, int D>
__global__ __launch_bounds__(64) void decode_split_kernel(const Params p) {
  constexpr int DP = 8;            // features per lane: one 16-byte piece of a row
  constexpr int PARTS = D / DP;    // lanes sharing one token row (16 or 8)
  constexpr int TPP = 64 / PARTS;  // tokens per pass (4 or 8)
  constexpr int PASSES = kBlock / TPP;
  static_assert(PARTS == 8 || PARTS == 16, "head dimension 64 or 128");

  const int lane = threadIdx.x;
  const int tok = lane / PARTS;
  const int part = lane % PARTS;
  const int split = blockIdx.x;
  const int hk = blockIdx.y / p.hgroups;
  const int h0 = hk * p.group + (blockIdx.y % p.hgroups) * GH;
  const int b = blockIdx.z;

  const int L = p.lens[b];
  if (L < 0 || L > p.max_blocks * kBlock) return;  // the combine writes NaN
  const int lo = split_lo_token(L, p.window);
  const int s_tok = split * kSplit;
  if (s_tok >= L || s_tok + kSplit <= lo) return;  // no visible token here

  // blocks of this split that hold visible tokens
  const int blk_first = max(s_tok, lo) / kBlock - split * kSplitBlocks;
  const int blk_last = min(kSplitBlocks, (L - s_tok + kBlock - 1) / kBlock);  // exclusive
  const int* trow = p.table + (int64_t)b * p.max_blocks + split * kSplitBlocks;
  const int64_t row_elems = (int64_t)p.Hkv * D;  // one token's row of the pool
  bool bad = false;

  // K/V registers of one block, [pass]: `ck/cv` are being computed while the
  // next block's loads land in `nk/nv`.  Only static indices, and no branch
  // around the loads, so that everything stays in registers.  A block id
  // outside the pool is replaced by block 0 (an in-bounds read) and the split
  // is flagged, which makes the whole sequence NaN.
  u32x4 ck[PASSES], cv[PASSES], nk[PASSES], nv[PASSES];
  auto fetch = [&](int i, u32x4 (&rk)[PASSES], u32x4 (&rv)[PASSES]) {
    int phys = trow[i];
    if (phys < 0 || phys >= p.num_blocks) {
      bad = true;
      phys = 0;
    }
    const int64_t base = ((int64_t)phys * kBlock) * row_elems + (int64_t)hk * D + part * DP;
#pragma unroll
    for (int pass = 0; pass < PASSES; ++pass) {
      const int64_t off = base + (int64_t)(pass * TPP + tok) * row_elems;
      rk[pass] = *reinterpret_cast<const u32x4*>(p.kc + off);
      rv[pass] = *reinterpret_cast<const u32x4*>(p.vc + off);
    }
  };
  // the first block's loads go out before the query's, so both latencies overlap
  if (blk_first < blk_last) fetch(blk_first, ck, cv);

  uint32_t qv[GH][4];
#pragma unroll
  for (int h = 0; h < GH; ++h) {
    const u32x4 x = *reinterpret_cast<const u32x4*>(p.q + ((int64_t)b * p.Hq + h0 + h) * D +
                                                    part * DP);
    qv[h][0] = x[0];
    qv[h][1] = x[1];
    qv[h][2] = x[2];
    qv[h][3] = x[3];
  }

  float m[GH], l[GH], acc[GH][DP];
#pragma unroll
  for (int h = 0; h < GH; ++h) {
    m[h] = kNegInf;
    l[h] = 0.f;
#pragma unroll
    for (int j = 0; j < DP; ++j) acc[h][j] = 0.f;
  }

  for (int i = blk_first; i < blk_last; ++i) {
    if (i + 1 < blk_last) fetch(i + 1, nk, nv);
#pragma unroll
    for (int pass = 0; pass < PASSES; ++pass) {
      const int t = s_tok + i * kBlock + pass * TPP + tok;
      const bool valid = t < L && t >= lo;
      float x[GH];
#pragma unroll
      for (int h = 0; h < GH; ++h) {
        float s = 0.f;
#pragma unroll
        for (int w = 0; w < 4; ++w)
          s = __builtin_amdgcn_fdot2_f32_bf16(as_bf16x2(qv[h][w]), as_bf16x2(ck[pass][w]), s, false);
        // all-reduce over the PARTS lanes of this token row
        s += dpp_f32<kDppXor1>(s);
        s += dpp_f32<kDppXor2>(s);
        s += dpp_f32<kDppHalfMirror>(s);
        if (PARTS == 16) s += dpp_f32<kDppRor8>(s);
        x[h] = valid ? s * p.sl2 : kNegInf;
      }
      bool need = false;
#pragma unroll
      for (int h = 0; h < GH; ++h) need = need || (x[h] > m[h] + kLazy);
      if (__builtin_amdgcn_ballot_w64(need) != 0) {
#pragma unroll
        for (int h = 0; h < GH; ++h) {
          const float mn = fmaxf(m[h], x[h]);
          const float a = (mn == kNegInf) ? 1.f : fast_exp2(m[h] - mn);
          m[h] = mn;
          l[h] *= a;
#pragma unroll
          for (int j = 0; j < DP; ++j) acc[h][j] *= a;
        }
      }
      float vf[DP];
#pragma unroll
      for (int w = 0; w < 4; ++w) {
        const uint32_t u = valid ? cv[pass][w] : 0u;  // tail slots may hold NaN
        vf[2 * w] = bf16lo_to_f32(u);
        vf[2 * w + 1] = bf16hi_to_f32(u);
      }
#pragma unroll
      for (int h = 0; h < GH; ++h) {
        const float pr = (x[h] == kNegInf) ? 0.f : fast_exp2(x[h] - m[h]);
        l[h] += pr;
#pragma unroll
        for (int j = 0; j < DP; ++j) acc[h][j] += pr * vf[j];
      }
    }
#pragma unroll
    for (int pass = 0; pass < PASSES; ++pass) {
      ck[pass] = nk[pass];
      cv[pass] = nv[pass];
    }
  }

  // merge the TPP token slots (lanes differing in the bits above PARTS) at a
  // common max
#pragma unroll
  for (int h = 0; h < GH; ++h) {
    float M = m[h];
#pragma unroll
    for (int o = PARTS; o < 64; o <<= 1) M = fmaxf(M, __shfl_xor(M, o, 64));
    const float f = (m[h] == kNegInf) ? 0.f : fast_exp2(m[h] - M);
    float ls = l[h] * f;
#pragma unroll
    for (int o = PARTS; o < 64; o <<= 1) ls += __shfl_xor(ls, o, 64);
#pragma unroll
    for (int j = 0; j < DP; ++j) {
      float a = acc[h][j] * f;
#pragma unroll
      for (int o = PARTS; o < 64; o <<= 1) a += __shfl_xor(a, o, 64);
      acc[h][j] = a;
    }
    m[h] = M;
    l[h] = ls;
  }
  const bool any_bad = __builtin_amdgcn_ballot_w64(bad) != 0;
  if (tok == 0) {
#pragma unroll
    for (int h = 0; h < GH; ++h) {
      const int64_t slot = ((int64_t)b * p.Hq + h0 + h) * p.max_splits + split;
      float* dst = p.ws_acc + slot * D + part * DP;
      f32x4 w0, w1;
      w0[0] = acc[h][0]; w0[1] = acc[h][1]; w0[2] = acc[h][2]; w0[3] = acc[h][3];
      w1[0] = acc[h][4]; w1[1] = acc[h][5]; w1[2] = acc[h][6]; w1[3] = acc[h][7];
      reinterpret_cast<f32x4*>(dst)[0] = w0;
      reinterpret_cast<f32x4*>(dst)[1] = w1;
      if (part == 0)
        p.ws_ml[slot] = any_bad ? make_float2(__builtin_nanf(""), __builtin_nanf(""))
                                : make_float2(m[h], l[h]);
    }
  }
}

template <int D>
__global__ __launch_bounds__(64 * kCombineWaves) void decode_combine_kernel(const Params p) {
  constexpr int PER = D / 64;  // features per lane
  __shared__ float red[kCombineWaves][D + 2];
  __shared__ float wmax[kCombineWaves];
  __shared__ int wbad[kCombineWaves];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int hq = blockIdx.x;
  const int b = blockIdx.y;
  const int64_t out_off = ((int64_t)b * p.Hq + hq) * D;

  const int L = p.lens[b];
  if (L < 0 || L > p.max_blocks * kBlock) {
    if (tid < D) p.o[out_off + tid] = 0x7fc0u;  // bf16 NaN
    if (tid == 0 && p.lse != nullptr) p.lse[(int64_t)b * p.Hq + hq] = __builtin_nanf("");
    return;
  }
  const int lo = split_lo_token(L, p.window);
  const int s0 = lo / kSplit;
  const int s1 = (L + kSplit - 1) / kSplit;
  const int64_t base = ((int64_t)b * p.Hq + hq) * p.max_splits;

  // common maximum and bad flag over all splits
  float M = kNegInf;
  int bad = 0;
  for (int s = s0 + tid; s < s1; s += 64 * kCombineWaves) {
    const float2 ml = p.ws_ml[base + s];
    if (ml.y != ml.y) bad = 1;
    M = fmaxf(M, ml.x);
  }
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) {
    M = fmaxf(M, __shfl_xor(M, o, 64));
    bad |= __shfl_xor(bad, o, 64);
  }
  if (lane == 0) {
    wmax[wave] = M;
    wbad[wave] = bad;
  }
  __syncthreads();
  M = wmax[0];
  bad = wbad[0];
#pragma unroll
  for (int w = 1; w < kCombineWaves; ++w) {
    M = fmaxf(M, wmax[w]);
    bad |= wbad[w];
  }

  float lsum = 0.f;
  float acc[PER];
#pragma unroll
  for (int j = 0; j < PER; ++j) acc[j] = 0.f;
  if (!bad && M != kNegInf) {
#pragma unroll 4
    for (int s = s0 + wave; s < s1; s += kCombineWaves) {
      const float2 ml = p.ws_ml[base + s];
      const float f = fast_exp2(ml.x - M);
      lsum += ml.y * f;
      const float* src = p.ws_acc + (base + s) * D + lane * PER;
#pragma unroll
      for (int j = 0; j < PER; ++j) acc[j] += src[j] * f;
    }
  }
#pragma unroll
  for (int j = 0; j < PER; ++j) red[wave][lane * PER + j] = acc[j];
  if (lane == 0) red[wave][D] = lsum;
  __syncthreads();
  if (wave == 0) {
    float lt = red[0][D];
#pragma unroll
    for (int w = 1; w < kCombineWaves; ++w) lt += red[w][D];
    const float inv = lt > 0.f ? 1.f / lt : 0.f;
#pragma unroll
    for (int j = 0; j < PER; ++j) {
      float a = red[0][lane * PER + j];
#pragma unroll
      for (int w = 1; w < kCombineWaves; ++w) a += red[w][lane * PER + j];
      const float o = bad ? __builtin_nanf("") : a * inv;
      bf16x2 v;
      v[0] = (__bf16)o;
      p.o[out_off + lane * PER + j] = __builtin_bit_cast(uint32_t, v) & 0xffffu;
    }
    if (lane == 0 && p.lse != nullptr)
      p.lse[(int64_t)b * p.Hq + hq] =
          bad ? __builtin_nanf("") : (lt > 0.f ? (M + log2f(lt)) * kLn2 : kNegInf);
  }
}

int max_splits_for(int block_size, int max_blocks_per_seq) {
  const long long tokens = (long long)block_size * max_blocks_per_seq;
  return (int)((tokens + kSplit - 1) / kSplit);
}

}  // namespace

size_t decode_workspace_bytes(int B, int Hq, int d, int block_size, int max_blocks_per_seq) {
  const size_t slots = (size_t)B * Hq * max_splits_for(block_size, max_blocks_per_seq);
  const size_t ml = (slots * sizeof(float2) + 255) / 256 * 256;
  return ml + slots * (size_t)d * sizeof(float);
}

template <int D>
static void launch_split(int gh, const Params& p, dim3 grid, hipStream_t s) {
  switch (gh) {
    case 8: hipLaunchKernelGGL((decode_split_kernel<8, D>), grid, dim3(64), 0, s, p); break;
    case 4: hipLaunchKernelGGL((decode_split_kernel<4, D>), grid, dim3(64), 0, s, p); break;
    case 2: hipLaunchKernelGGL((decode_split_kernel<2, D>), grid, dim3(64), 0, s, p); break;
    default: hipLaunchKernelGGL((decode_split_kernel<1, D>), grid, dim3(64), 0, s, p); break;
  }
}

hipError_t launch_decode_paged(const DecodeArgs& a, hipStream_t stream) {
  if (a.B == 0) return hipSuccess;
  const int G = a.Hq / a.Hkv;
  const int gh = (G % 8 == 0) ? 8 : (G % 4 == 0) ? 4 : (G % 2 == 0) ? 2 : 1;
  Params p;
  p.q = static_cast<const uint16_t*>(a.q);
  p.kc = static_cast<const uint16_t*>(a.kcache);
  p.vc = static_cast<const uint16_t*>(a.vcache);
  p.table = a.block_table;
  p.lens = a.seq_lens;
  p.o = static_cast<uint16_t*>(a.out);
  p.lse = a.lse;
  p.Hq = a.Hq;
  p.Hkv = a.Hkv;
  p.group = G;
  p.hgroups = G / gh;
  p.max_blocks = a.max_blocks_per_seq;
  p.num_blocks = a.num_blocks;
  p.window = a.window;
  p.max_splits = max_splits_for(a.block_size, a.max_blocks_per_seq);
  p.sl2 = a.scale * kLog2e;
  const size_t slots = (size_t)a.B * a.Hq * p.max_splits;
  const size_t ml_bytes = (slots * sizeof(float2) + 255) / 256 * 256;
  p.ws_ml = static_cast<float2*>(a.workspace);
  p.ws_acc = reinterpret_cast<float*>(static_cast<char*>(a.workspace) + ml_bytes);

  const dim3 grid1(p.max_splits, a.Hkv * p.hgroups, a.B);
  if (a.d == 128)
    launch_split<128>(gh, p, grid1, stream);
  else
    launch_split<64>(gh, p, grid1, stream);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  const dim3 grid2(a.Hq, a.B);
  if (a.d == 128)
    hipLaunchKernelGGL(decode_combine_kernel<128>, grid2, dim3(64 * kCombineWaves), 0, stream, p);
  else
    hipLaunchKernelGGL(decode_combine_kernel<64>, grid2, dim3(64 * kCombineWaves), 0, stream, p);
  return hipGetLastError();
}

}  // namespace attn
