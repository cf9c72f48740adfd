// Single-query decode over a block-paged KV cache, split along the keys.
//
// Method: a decode step's one new query reads every cached K/V of its
// sequence ("Ch. 3: MHA Limitations, MQA, GQA, and FlashAttention", 3.1);
// the cache is split into fixed-size blocks reached through a lookup table
// ("Inference Engineering", 2.5); the keys are cut into pieces whose partial
// softmax states (m, l, acc) are merged exactly afterwards (the rescale of
// "Ch. 3", 3.5: l e^m is invariant, so states rescaled to a common maximum
// add).
//
// Work split.  All cache blocks the batch reads are laid end to end, sequence
// after sequence, and cut into W equal ranges, so every wave streams the same
// number of blocks whatever the length mix; a range that crosses a sequence
// boundary yields one partial state per sequence it touches.  A wave serves
// one KV head and up to 16 of the query heads that share it.  The waves of a
// work group take the same range for up to 8 consecutive (KV head, head
// group) pairs, so they read the same cache blocks side by side: a block's
// token rows hold all KV heads next to each other, and the group's waves
// together read them whole and at the same time.
//
// Kernel 1 (split), per 16-token block, all on the matrix cores:
//   S^T = K Q^T   v_mfma_f32_16x16x32_bf16, A = 16 key rows straight from
//                 memory (lane (n, g): token n, features 32c + 8g .. +8),
//                 B = the query heads' rows (lane column n = head);
//   softmax       lane (n, g) holds tokens 4g .. 4g+3 of head n: the block max
//                 is in-lane; the running max is raised lazily (only when a
//                 score passes it by more than 2^8), equal on a head's 4 lanes;
//   O^T += V^T P^T  v_mfma_f32_16x16x16_bf16, B = the lane's own 4
//                 probabilities (bf16, round to nearest even), A = V^T read
//                 with the transposing LDS load from the block's V rows, which
//                 the wave stages in its own LDS slot.
// The next block's K/V loads are in flight while a block is computed; they are
// non-temporal loads (the cache is streamed once per call).
//
// Kernel 2 (combine): one work group per (sequence, query head); 4 waves each
// take every 4th partial, rescale to the common maximum and sum in a fixed
// order; the 4 partial sums are added in LDS.  Deterministic: no atomics.
#include <atomic>

#include "device_common.h"
#include "launch.h"

namespace attn {
namespace {

constexpr int kBlock = 16;         // tokens per cache block
constexpr float kLazy = 8.0f;      // rescale only when a score passes max + 8 (base 2)
constexpr int kCombineWaves = 4;
constexpr int kMaxRanges = 512;    // block ranges (work groups along x): bounds the workspace
constexpr int kWavesPerSimd = 2;   // resident split waves per SIMD (register bound)
constexpr int kGroupWaves = 8;     // most (KV head, head group) pairs in one work group

typedef short s16x4 __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) s16x4 lds_s16x4;

struct Params {
  const uint16_t* q;
  const uint16_t* kc;
  const uint16_t* vc;
  const int* table;
  const int* lens;
  uint16_t* o;
  float* lse;
  float2* ws_ml;   // [Hq, kMaxRanges + B] (m, l); slot of (range w, sequence b) = w + b
  float* ws_acc;   // [Hq, kMaxRanges + B, D]
  int2* ws_seq;    // [B] (first range, last range) covering the sequence
  int B, Hq, Hkv, group, hgroups, max_blocks, num_blocks, window, W, slots;
  int pairs, gwaves;  // (KV head, head group) pairs, and pairs per work group
  float sl2;
};

// Cache blocks a sequence of length L reads (0 for a length the kernels reject).
__device__ __forceinline__ int seq_blocks(int L, int max_blocks, int window) {
  if (L <= 0 || L > max_blocks * kBlock) return 0;
  const int lo = window > 0 ? max(0, L - window) : 0;
  return (L + kBlock - 1) / kBlock - lo / kBlock;
}

__device__ __forceinline__ int lo_token(int L, int window) {
  return window > 0 ? max(0, L - window) : 0;
}

template <int D>
struct DecTile {
  static constexpr int KC = D / 32;       // 16x16x32 products over the head dimension
  static constexpr int NT = D / 16;       // 16-feature tiles of O^T
  static constexpr int RL = D / 8;        // lanes per token row in a V load (16 bytes each)
  static constexpr int RPI = 64 / RL;     // token rows per V load instruction
  static constexpr int VI = kBlock / RPI; // V load instructions per block
  static constexpr int PITCH = D + 16;    // LDS row pitch (bf16): rows fall 32 bytes apart mod 256
};

template <int D>
__global__ __launch_bounds__(64 * kGroupWaves) void decode_split_kernel(const Params p) {
  using T = DecTile<D>;
  __shared__ __attribute__((aligned(16))) uint16_t vs_all[kGroupWaves][kBlock * T::PITCH];

  const int lane = threadIdx.x & 63;
  const int wv = threadIdx.x >> 6;
  const int pair = blockIdx.y * p.gwaves + wv;  // (KV head, head group) of this wave
  if (pair >= p.pairs) return;  // no barriers below: the group's waves are independent
  uint16_t* const vs = vs_all[wv];
  const int n = lane & 15;   // MFMA column: query head; also the K token row
  const int g = lane >> 4;   // MFMA k-group
  const int w = blockIdx.x;
  const int hk = pair / p.hgroups;
  const int hsub = (pair % p.hgroups) * 16;  // first head of this wave within the group
  const int nh = min(16, p.group - hsub);          // heads this wave serves
  const int h0 = hk * p.group + hsub;

  // Blocks of all sequences laid end to end: C_b = blocks before sequence b,
  // T = all blocks.  A wave-wide prefix sum, 64 sequences at a time, finds the
  // total and the sequence holding this wave's first block.
  int total = 0;  // (the same in every wave of the grid)
  for (int c = 0; c < p.B; c += 64) {
    const int j = c + lane;
    int x = j < p.B ? seq_blocks(p.lens[j], p.max_blocks, p.window) : 0;
#pragma unroll
    for (int o = 32; o >= 1; o >>= 1) x += __shfl_xor(x, o, 64);
    total += x;
  }
  // never more ranges than blocks, so that every range owns at least one block
  // and the ranges covering a sequence are consecutive and all write a partial
  const int nw = min(p.W, total);
  if (w >= nw) return;
  const int g0 = (int)((int64_t)w * total / nw);
  const int g1 = (int)((int64_t)(w + 1) * total / nw);
  int b = 0, cb = 0;  // first sequence touching [g0, g1) and its C_b
  for (int c = 0; c < p.B; c += 64) {
    const int j = c + lane;
    const int x = j < p.B ? seq_blocks(p.lens[j], p.max_blocks, p.window) : 0;
    int incl = x;
#pragma unroll
    for (int o = 1; o < 64; o <<= 1) {
      const int y = __shfl_up(incl, o, 64);
      if (lane >= o) incl += y;
    }
    incl += cb;
    const uint64_t hit = __builtin_amdgcn_ballot_w64(incl > g0);
    if (hit != 0) {
      const int f = __builtin_ctzll(hit);
      b = c + f;
      cb = __shfl(incl - x, f, 64);
      break;
    }
    cb = __shfl(incl, 63, 64);
  }

  const int64_t row_elems = (int64_t)p.Hkv * D;
  // per-lane element offsets inside a block of the pool
  const int64_t koff = (int64_t)n * row_elems + hk * D + 8 * g;  // K: token n, 8 features
  const int vrow = lane / T::RL;
  const int vcol = 8 * (lane % T::RL);
  const int64_t voff = (int64_t)vrow * row_elems + hk * D + vcol;
  const uint32_t vs_base = (uint32_t)(uintptr_t)vs;  // this wave's staging rows
  const int sl = lane & 15;
  // transposing-read address: lane (sl, g) supplies row 4g + sl/4, features 4(sl%4) ..+3
  const uint32_t rd = vs_base + 2u * (uint32_t)((4 * g + (sl >> 2)) * T::PITCH + 4 * (sl & 3));

  int gpos = g0;
  while (gpos < g1) {
    const int L = p.lens[b];
    const int nb = seq_blocks(L, p.max_blocks, p.window);
    const int end = min(g1, cb + nb);
    if (gpos >= end) {  // an empty sequence: nothing to read
      cb += nb;
      ++b;
      continue;
    }
    const int lo = lo_token(L, p.window);
    const int first_blk = lo / kBlock + (gpos - cb);   // block index within the sequence
    const int count = end - gpos;
    const int* trow = p.table + (int64_t)b * p.max_blocks + first_blk;
    bool bad = false;

    // K as the A operand of S^T = K Q^T and V rows (RPI rows an instruction);
    // two register sets, filled alternately.
    u32x4 kA[T::KC], kB[T::KC], vA[T::VI], vB[T::VI];
    // block ids are read two blocks ahead of their fetch (scalar loads whose
    // latency would otherwise sit in front of every block's K/V loads)
    auto fetch = [&](int id, u32x4 (&rk)[T::KC], u32x4 (&rv)[T::VI]) {
      int phys = id;
      if (phys < 0 || phys >= p.num_blocks) {
        bad = true;
        phys = 0;
      }
      const int64_t base = (int64_t)phys * kBlock * row_elems;
      const uint16_t* kp = p.kc + base + koff;
      const uint16_t* vp = p.vc + base + voff;
      // non-temporal: the cache is read once per call, so its lines should not
      // displace (or force the write-back of) what the caches hold
#pragma unroll
      for (int c = 0; c < T::KC; ++c)
        rk[c] = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(kp + 32 * c));
#pragma unroll
      for (int j = 0; j < T::VI; ++j)
        rv[j] = __builtin_nontemporal_load(
            reinterpret_cast<const u32x4*>(vp + (int64_t)j * T::RPI * row_elems));
    };
    int id_b = trow[min(1, count - 1)], id_c = trow[min(2, count - 1)];
    fetch(trow[0], kA, vA);

    // Q^T as the B operand: lane (n, g) holds head n, the same features as K
    bf16x8 qf[T::KC];
#pragma unroll
    for (int c = 0; c < T::KC; ++c) {
      u32x4 x = {0u, 0u, 0u, 0u};
      if (n < nh)
        x = *reinterpret_cast<const u32x4*>(p.q + ((int64_t)b * p.Hq + h0 + n) * D + 32 * c + 8 * g);
      qf[c] = __builtin_bit_cast(bf16x8, x);
    }

    // O^T tiles (16 features x 16 heads): lane (n, g) holds features 16t + 4g + r
    // of head n.  m is equal on the four lanes of a head; l is a per-lane partial sum.
    f32x4 acc[T::NT];
#pragma unroll
    for (int t = 0; t < T::NT; ++t) acc[t] = f32x4{0.f, 0.f, 0.f, 0.f};
    float m = kNegInf, mth = kNegInf, lsum = 0.f;

    auto compute = [&](int i, const u32x4 (&rk)[T::KC], const u32x4 (&rv)[T::VI]) {
      const int t0 = (first_blk + i) * kBlock;             // first token of the block
      const bool edge = (t0 < lo) || (t0 + kBlock > L);    // wave-uniform
      // V rows to LDS (tokens outside [lo, L) as zeros: their slots may hold NaN)
#pragma unroll
      for (int j = 0; j < T::VI; ++j) {
        u32x4 v = rv[j];
        if (edge) {
          const int tk = t0 + j * T::RPI + vrow;
          if (tk < lo || tk >= L) v = u32x4{0u, 0u, 0u, 0u};
        }
        *reinterpret_cast<u32x4*>(&vs[(j * T::RPI + vrow) * T::PITCH + vcol]) = v;
      }
      // S^T: lane (n, g) gets tokens 4g + r of head n
      f32x4 s = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int c = 0; c < T::KC; ++c)
        s = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, rk[c]), qf[c], s, 0, 0, 0);
      float x[4];
#pragma unroll
      for (int r = 0; r < 4; ++r) x[r] = s[r] * p.sl2;
      if (edge) {
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          const int tk = t0 + 4 * g + r;
          if (tk < lo || tk >= L) x[r] = kNegInf;
        }
      }
      float mx = fmaxf(fmaxf(x[0], x[1]), fmaxf(x[2], x[3]));
      float a = 1.f;
      if (__builtin_amdgcn_ballot_w64(mx > mth) != 0) {
        // raise the head's maximum (the same on its four lanes)
        mx = fmaxf(mx, __shfl_xor(mx, 16, 64));
        mx = fmaxf(mx, __shfl_xor(mx, 32, 64));
        const float mn = fmaxf(m, mx);
        a = (mn == kNegInf) ? 1.f : fast_exp2(m - mn);
        m = mn;
        mth = mn + kLazy;
      }
      // unconditional (a == 1 almost always): keeps the accumulators out of the branch
      lsum *= a;
#pragma unroll
      for (int t = 0; t < T::NT; ++t) acc[t] *= a;
      float pr[4];
#pragma unroll
      for (int r = 0; r < 4; ++r) pr[r] = fast_exp2(x[r] - m);
      if (edge) {
#pragma unroll
        for (int r = 0; r < 4; ++r) pr[r] = (x[r] == kNegInf) ? 0.f : pr[r];
      }
      lsum += (pr[0] + pr[1]) + (pr[2] + pr[3]);
      u32x2 pw;
      pw[0] = pack_bf16x2(pr[0], pr[1]);
      pw[1] = pack_bf16x2(pr[2], pr[3]);
      const s16x4 pb = __builtin_bit_cast(s16x4, pw);
      // O^T += V^T P^T: the transposing LDS read gives lane (n, g) tokens
      // 4g .. 4g+3 of feature 16t + n
#pragma unroll
      for (int t = 0; t < T::NT; ++t) {
        const s16x4 va = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4*)(uintptr_t)(rd + 32u * t));
        acc[t] = __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(va, pb, acc[t], 0, 0, 0);
      }
    };

    // The prefetch index is clamped, so the last block is read twice (the
    // second time from cache) rather than branching around the loads.
    for (int i = 0; i < count; i += 2) {
      // ids of blocks i+3 and i+4 for the next trip; id_b, id_c: blocks i+1, i+2
      const int id_d = trow[min(i + 3, count - 1)], id_e = trow[min(i + 4, count - 1)];
      fetch(id_b, kB, vB);
      compute(i, kA, vA);
      if (i + 1 >= count) break;
      fetch(id_c, kA, vA);
      compute(i + 1, kB, vB);
      id_b = id_d;
      id_c = id_e;
    }

    // l over the four lanes of each head; one partial per (wave, sequence)
    lsum += __shfl_xor(lsum, 16, 64);
    lsum += __shfl_xor(lsum, 32, 64);
    const bool any_bad = __builtin_amdgcn_ballot_w64(bad) != 0;
    if (n < nh) {
      const int64_t slot = (int64_t)(h0 + n) * p.slots + w + b;
      float* dst = p.ws_acc + slot * D + 4 * g;
#pragma unroll
      for (int t = 0; t < T::NT; ++t) *reinterpret_cast<f32x4*>(dst + 16 * t) = acc[t];
      if (g == 0)
        p.ws_ml[slot] = any_bad ? make_float2(__builtin_nanf(""), __builtin_nanf(""))
                                : make_float2(m, lsum);
    }
    // the ranges holding a sequence's first and last blocks record themselves
    if (pair == 0 && lane == 0) {
      if (gpos == cb) p.ws_seq[b].x = w;
      if (end == cb + nb) p.ws_seq[b].y = w;
    }
    gpos = end;
    cb += nb;
    ++b;
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
  // partials of this sequence: slots w + b for the ranges w that covered it
  int s0 = 0, s1 = 0;
  if (seq_blocks(L, p.max_blocks, p.window) > 0) {
    const int2 fl = p.ws_seq[b];
    s0 = max(0, fl.x + b);
    s1 = min(p.slots, fl.y + b + 1);
  }
  const int64_t base = (int64_t)hq * p.slots;

  // common maximum and bad flag over all partials
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


}  // namespace

size_t decode_workspace_bytes(int B, int Hq, int d, int block_size, int max_blocks_per_seq) {
  (void)block_size;
  (void)max_blocks_per_seq;
  const size_t slots = (size_t)Hq * (kMaxRanges + B);
  const size_t seq = ((size_t)B * sizeof(int2) + 255) / 256 * 256;
  const size_t ml = (slots * sizeof(float2) + 255) / 256 * 256;
  return seq + ml + slots * (size_t)d * sizeof(float);
}

hipError_t launch_decode_paged(const DecodeArgs& a, hipStream_t stream) {
  if (a.B == 0) return hipSuccess;
  const int G = a.Hq / a.Hkv;
  Params p;
  p.q = static_cast<const uint16_t*>(a.q);
  p.kc = static_cast<const uint16_t*>(a.kcache);
  p.vc = static_cast<const uint16_t*>(a.vcache);
  p.table = a.block_table;
  p.lens = a.seq_lens;
  p.o = static_cast<uint16_t*>(a.out);
  p.lse = a.lse;
  p.B = a.B;
  p.Hq = a.Hq;
  p.Hkv = a.Hkv;
  p.group = G;
  p.hgroups = (G + 15) / 16;
  p.max_blocks = a.max_blocks_per_seq;
  p.num_blocks = a.num_blocks;
  p.window = a.window;
  p.sl2 = a.scale * kLog2e;
  // one wave per resident slot of the whole GPU: W block ranges, each taken by
  // ceil(pairs / gwaves) work groups of up to 8 waves
  p.pairs = a.Hkv * p.hgroups;
  p.gwaves = p.pairs < kGroupWaves ? p.pairs : kGroupWaves;
  const int ygroups = (p.pairs + p.gwaves - 1) / p.gwaves;
  const int resident = device_cus() * 4 * kWavesPerSimd;
  p.W = max(1, min(kMaxRanges, resident / (p.gwaves * ygroups)));
  p.slots = kMaxRanges + a.B;
  char* ws = static_cast<char*>(a.workspace);
  const size_t seq_bytes = ((size_t)a.B * sizeof(int2) + 255) / 256 * 256;
  const size_t slots = (size_t)a.Hq * p.slots;
  const size_t ml_bytes = (slots * sizeof(float2) + 255) / 256 * 256;
  p.ws_seq = reinterpret_cast<int2*>(ws);
  p.ws_ml = reinterpret_cast<float2*>(ws + seq_bytes);
  p.ws_acc = reinterpret_cast<float*>(ws + seq_bytes + ml_bytes);

  const dim3 grid1(p.W, ygroups);
  if (a.d == 128)
    hipLaunchKernelGGL(decode_split_kernel<128>, grid1, dim3(64 * p.gwaves), 0, stream, p);
  else
    hipLaunchKernelGGL(decode_split_kernel<64>, grid1, dim3(64 * p.gwaves), 0, stream, p);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  const dim3 grid2(a.Hq, a.B);
  if (a.d == 128)
    hipLaunchKernelGGL(decode_combine_kernel<128>, grid2, dim3(64 * kCombineWaves), 0, stream, p);
  else
    hipLaunchKernelGGL(decode_combine_kernel<64>, grid2, dim3(64 * kCombineWaves), 0, stream, p);
  return hipGetLastError();
}

// ---- Decode without a caller workspace.  The partials live in this file's
// own device array (each GPU the library runs on holds one, from module load
// until the process ends).  Host code never passes the array's name to a
// kernel: that name is a host-side stand-in, not a device address.  The first
// call on each device looks the address up with hipGetSymbolAddress (that
// device current) and keeps it; every later call uses the kept pointer.
// Nothing in the array needs to start at zero (the kernels write every value
// they read), and all calls on one GPU share it, so calls that overlap on one
// GPU race.

namespace {
constexpr size_t kScratchBytes = size_t(16) << 20;  // 16 MiB per device
static __device__ __align__(256) unsigned char scratch[kScratchBytes];
constexpr int kMaxDevices = 64;
std::atomic<void*> g_scratch_ptr[kMaxDevices];
}  // namespace

size_t decode_scratch_bytes() { return kScratchBytes; }

hipError_t launch_decode_paged_noalloc(const DecodeArgs& args, hipStream_t stream) {
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
  void* ptr = g_scratch_ptr[dev].load(std::memory_order_acquire);
  if (ptr == nullptr) {
    // racing first calls on one device store the same address
    e = hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch));
    if (e != hipSuccess) return e;
    if (ptr == nullptr) return hipErrorInvalidSymbol;
    g_scratch_ptr[dev].store(ptr, std::memory_order_release);
  }
  DecodeArgs a = args;
  a.workspace = ptr;
  return launch_decode_paged(a, stream);
}

}  // namespace attn
