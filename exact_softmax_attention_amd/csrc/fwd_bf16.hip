// Tiled, fused prefill/training forward for bf16 Q/K/V on gfx950.
//
// The loop is the one of "Attention Is O(n^2): FlashAttention vs Linear
// Attention" (section "FlashAttention - Same FLOPs, Linear Memory"): each
// work group owns a block of query rows, walks the key/value tiles once,
// keeps a running row maximum and row sum, rescales its accumulator when the
// maximum grows, and divides by the sum at the end; the log-sum-exp is written
// for a backward pass.  Score and probability tiles live only in registers.
//
// MI355X mapping (this library's own design):
//   * 4 waves x 32 query rows = 128 rows per work group.  Each wave computes
//     S^T = K Q^T with v_mfma_f32_32x32x16_bf16 (A = K rows from LDS, B = its
//     Q rows held in registers for the whole loop).  In the 32x32 accumulator
//     layout lane l holds column l % 32, i.e. one query row, and 16 keys, so
//     the row max / row sum are in-lane plus one exchange with lane l ^ 32.
//   * O^T = V^T P^T, again 32x32x16: B = P^T straight from the score
//     registers (converted to bf16, round-to-nearest-even), A = V^T read from
//     an LDS copy of V stored transposed (keys contiguous per feature).  The
//     key order inside each 16-key chunk is permuted so that every lane's 8
//     keys of P match one 16-byte LDS read of V^T; the contraction does not
//     care about the order as long as both operands agree.
//   * K/V tiles are staged global -> registers -> LDS with two LDS buffers:
//     the next tile's global loads are in flight while the current tile is
//     computed.  Tiles wholly outside the causal/window band are never
//     visited; only tiles that cut the band boundary or the key tail pay for
//     the per-element mask.
//   * Work groups are ordered heavy-first (last query tiles first) inside a
//     head and remapped so that the tiles of one head share an XCD (and its
//     L2), since they all stream the same K/V.
#include "device_common.h"
#include "launch.h"

namespace attn {
namespace {

constexpr int kWaves = 4;
constexpr int kRowsPerWave = 32;
constexpr int kBM = kWaves * kRowsPerWave;  // query rows per work group
constexpr int kThreads = kWaves * 64;

template <int D>
struct Tile {
  static constexpr int BN = (D == 128) ? 64 : 128;  // keys per tile
  static constexpr int NKB = BN / 32;                // 32-key blocks of S^T
  static constexpr int NDB = D / 32;                 // 32-feature blocks of O^T
  static constexpr int KC = D / 16;                  // k-chunks of K Q^T
  static constexpr int VC = BN / 16;                 // k-chunks of V^T P^T
  static constexpr int KSTRIDE = D + 8;              // bf16 per K row in LDS
  static constexpr int VSTRIDE = BN + 8;             // bf16 per V^T row in LDS
  static constexpr int K_ELEMS = BN * KSTRIDE;
  static constexpr int V_ELEMS = D * VSTRIDE;
  static constexpr int STAGE = K_ELEMS + V_ELEMS;
  static constexpr int K_CHUNKS = BN * D / 8 / kThreads;  // 16-byte K pieces per thread
  static constexpr int V_ITEMS = BN * D / 32 / kThreads;  // (4 keys x 8 features) per thread
  static_assert(K_CHUNKS * kThreads * 8 == BN * D, "K staging must cover the tile");
  static_assert(V_ITEMS * kThreads * 32 == BN * D, "V staging must cover the tile");
};

struct Params {
  const uint16_t* q;
  const uint16_t* k;
  const uint16_t* v;
  uint16_t* o;
  float* lse;
  int Hq, Hkv, group, Nq, Nk, causal, window, n_qtiles, total;
  float sl2;  // scale * log2(e): scores are kept in the base-2 domain
};

// Position of key `key16` (0..15) of a 16-key chunk inside the transposed V
// tile.  Key a*8 + g*4 + e goes to g*8 + a*4 + e: lane group g of the P^T
// operand holds exactly keys {g*4 .. g*4+3, 8+g*4 .. 8+g*4+3} of each chunk.
__device__ __forceinline__ int vt_pos(int key) {
  const int chunk = key >> 4, k16 = key & 15;
  const int a = k16 >> 3, gg = (k16 >> 2) & 1, e = k16 & 3;
  return chunk * 16 + gg * 8 + a * 4 + e;
}

template <int D>
__global__ __launch_bounds__(kThreads, 2) void fwd_bf16_kernel(const Params p) {
  using T = Tile<D>;
  __shared__ __attribute__((aligned(16))) uint16_t smem[2 * T::STAGE];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int n = lane & 31;  // query row within the wave / MFMA column
  const int g = lane >> 5;  // k-half of the MFMA operands

  const int item = xcd_remap(blockIdx.x, p.total);
  const int bh = item / p.n_qtiles;
  const int qt = p.n_qtiles - 1 - (item - bh * p.n_qtiles);
  const int b = bh / p.Hq;
  const int h = bh - b * p.Hq;
  const int hk = h / p.group;
  const int i0 = qt * kBM;
  const int qw0 = i0 + wave * kRowsPerWave;
  const int delta = p.Nk - p.Nq;

  int kv_end = p.Nk;
  if (p.causal) kv_end = min(p.Nk, i0 + kBM + delta);
  int kv_begin = 0;
  if (p.window > 0) kv_begin = max(0, i0 + delta - p.window + 1);
  const int t_begin = kv_begin / T::BN;
  const int t_end = kv_end > kv_begin ? (kv_end + T::BN - 1) / T::BN : t_begin;

  // this wave's Q rows as the B operand of K Q^T (8 bf16 per k-chunk)
  const int64_t q_row = (int64_t)p.Hq * D;
  bf16x8 qf[T::KC];
  {
    const int row = qw0 + n;
    if (row < p.Nq) {
      const uint16_t* qp = p.q + ((int64_t)b * p.Nq + row) * q_row + (int64_t)h * D + g * 8;
#pragma unroll
      for (int c = 0; c < T::KC; ++c) qf[c] = *reinterpret_cast<const bf16x8*>(qp + c * 16);
    } else {
#pragma unroll
      for (int c = 0; c < T::KC; ++c) qf[c] = bf16x8{};
    }
  }

  const int64_t kv_row = (int64_t)p.Hkv * D;
  const uint16_t* kbase = p.k + (int64_t)b * p.Nk * kv_row + (int64_t)hk * D;
  const uint16_t* vbase = p.v + (int64_t)b * p.Nk * kv_row + (int64_t)hk * D;

  u32x4 kreg[T::K_CHUNKS];
  u32x4 vreg[4 * T::V_ITEMS];

  auto load_tile = [&](int t) {
    const int j0 = t * T::BN;
#pragma unroll
    for (int c = 0; c < T::K_CHUNKS; ++c) {
      const int cid = tid + c * kThreads;
      const int row = cid / (D / 8);
      const int col = cid % (D / 8);
      const int j = j0 + row;
      kreg[c] = (j < p.Nk) ? *reinterpret_cast<const u32x4*>(kbase + (int64_t)j * kv_row + col * 8)
                           : u32x4{0u, 0u, 0u, 0u};
    }
#pragma unroll
    for (int i = 0; i < T::V_ITEMS; ++i) {
      const int it = tid + i * kThreads;
      const int dc = it % (D / 8);
      const int kg = it / (D / 8);
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const int j = j0 + kg * 4 + e;
        vreg[i * 4 + e] = (j < p.Nk)
            ? *reinterpret_cast<const u32x4*>(vbase + (int64_t)j * kv_row + dc * 8)
            : u32x4{0u, 0u, 0u, 0u};
      }
    }
  };

  auto store_tile = [&](int buf) {
    uint16_t* ks = smem + buf * T::STAGE;
    uint16_t* vs = ks + T::K_ELEMS;
#pragma unroll
    for (int c = 0; c < T::K_CHUNKS; ++c) {
      const int cid = tid + c * kThreads;
      const int row = cid / (D / 8);
      const int col = cid % (D / 8);
      *reinterpret_cast<u32x4*>(ks + row * T::KSTRIDE + col * 8) = kreg[c];
    }
#pragma unroll
    for (int i = 0; i < T::V_ITEMS; ++i) {
      const int it = tid + i * kThreads;
      const int dc = it % (D / 8);
      const int kg = it / (D / 8);
      const int pos = vt_pos(kg * 4);
      const u32x4 v0 = vreg[i * 4 + 0], v1 = vreg[i * 4 + 1];
      const u32x4 v2 = vreg[i * 4 + 2], v3 = vreg[i * 4 + 3];
#pragma unroll
      for (int w = 0; w < 4; ++w) {
        // features 2w (low halves) and 2w+1 (high halves) of the 4 keys
        u32x2 lo, hi;
        lo[0] = (v0[w] & 0xffffu) | (v1[w] << 16);
        lo[1] = (v2[w] & 0xffffu) | (v3[w] << 16);
        hi[0] = (v0[w] >> 16) | (v1[w] & 0xffff0000u);
        hi[1] = (v2[w] >> 16) | (v3[w] & 0xffff0000u);
        *reinterpret_cast<u32x2*>(vs + (dc * 8 + 2 * w) * T::VSTRIDE + pos) = lo;
        *reinterpret_cast<u32x2*>(vs + (dc * 8 + 2 * w + 1) * T::VSTRIDE + pos) = hi;
      }
    }
  };

  float m_run = kNegInf;  // running row max (base-2 domain), same in lanes n and n+32
  float l_run = 0.f;      // running row sum over this lane's keys
  f32x16 acc[T::NDB];
#pragma unroll
  for (int db = 0; db < T::NDB; ++db) acc[db] = f32x16{};

  if (t_begin < t_end) {
    load_tile(t_begin);
    store_tile(0);
  }
  __syncthreads();

  for (int t = t_begin; t < t_end; ++t) {
    const int buf = (t - t_begin) & 1;
    const bool has_next = t + 1 < t_end;
    if (has_next) load_tile(t + 1);
    const int j0 = t * T::BN;

    bool skip = qw0 >= p.Nq;
    if (p.causal && j0 > qw0 + kRowsPerWave - 1 + delta) skip = true;
    if (p.window > 0 && j0 + T::BN - 1 < qw0 + delta - p.window + 1) skip = true;

    if (!skip) {
      const uint16_t* ks = smem + buf * T::STAGE;
      const uint16_t* vs = ks + T::K_ELEMS;

      // S^T = K Q^T for the tile's NKB blocks of 32 keys
      f32x16 st[T::NKB];
#pragma unroll
      for (int kb = 0; kb < T::NKB; ++kb) {
        st[kb] = f32x16{};
#pragma unroll
        for (int c = 0; c < T::KC; ++c) {
          const bf16x8 kf =
              *reinterpret_cast<const bf16x8*>(ks + (kb * 32 + n) * T::KSTRIDE + c * 16 + g * 8);
          st[kb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(kf, qf[c], st[kb], 0, 0, 0);
        }
      }

      // scale into the base-2 domain; mask only tiles that cut the band or the tail
      const bool need_mask = (j0 + T::BN > p.Nk) ||
                             (p.causal && j0 + T::BN - 1 > qw0 + delta) ||
                             (p.window > 0 && qw0 + kRowsPerWave - 1 + delta - j0 >= p.window);
#pragma unroll
      for (int kb = 0; kb < T::NKB; ++kb)
#pragma unroll
        for (int r = 0; r < 16; ++r) st[kb][r] *= p.sl2;
      if (need_mask) {
        const int pos = qw0 + n + delta;
#pragma unroll
        for (int kb = 0; kb < T::NKB; ++kb)
#pragma unroll
          for (int r = 0; r < 16; ++r) {
            const int key = j0 + kb * 32 + (r >> 2) * 8 + g * 4 + (r & 3);
            bool vis = key < p.Nk;
            if (p.causal) vis = vis && key <= pos;
            if (p.window > 0) vis = vis && (pos - key) < p.window;
            if (!vis) st[kb][r] = kNegInf;
          }
      }

      // online softmax update
      float mx = kNegInf;
#pragma unroll
      for (int kb = 0; kb < T::NKB; ++kb)
#pragma unroll
        for (int r = 0; r < 16; ++r) mx = fmaxf(mx, st[kb][r]);
      mx = fmaxf(mx, swap_halves(mx));
      const float m_new = fmaxf(m_run, mx);
      const float m_use = (m_new == kNegInf) ? 0.f : m_new;  // row with nothing visible yet
      const float alpha = fast_exp2(m_run - m_use);
      m_run = m_new;

      uint32_t pk[T::NKB][8];
      float rs = 0.f;
#pragma unroll
      for (int kb = 0; kb < T::NKB; ++kb)
#pragma unroll
        for (int i = 0; i < 8; ++i) {
          const float p0 = fast_exp2(st[kb][2 * i] - m_use);
          const float p1 = fast_exp2(st[kb][2 * i + 1] - m_use);
          const uint32_t w = pack_bf16x2(p0, p1);
          pk[kb][i] = w;
          rs += bf16lo_to_f32(w) + bf16hi_to_f32(w);  // the sum of what the MFMA sees
        }
      l_run = l_run * alpha + rs;
#pragma unroll
      for (int db = 0; db < T::NDB; ++db)
#pragma unroll
        for (int r = 0; r < 16; ++r) acc[db][r] *= alpha;

      // O^T += V^T P^T
#pragma unroll
      for (int kc = 0; kc < T::VC; ++kc) {
        const int kb = kc >> 1, half = kc & 1;
        u32x4 pw;
        pw[0] = pk[kb][half * 4 + 0];
        pw[1] = pk[kb][half * 4 + 1];
        pw[2] = pk[kb][half * 4 + 2];
        pw[3] = pk[kb][half * 4 + 3];
        const bf16x8 pb = __builtin_bit_cast(bf16x8, pw);
#pragma unroll
        for (int db = 0; db < T::NDB; ++db) {
          const bf16x8 vf =
              *reinterpret_cast<const bf16x8*>(vs + (db * 32 + n) * T::VSTRIDE + kc * 16 + g * 8);
          acc[db] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(vf, pb, acc[db], 0, 0, 0);
        }
      }
    }

    if (has_next) store_tile(buf ^ 1);
    __syncthreads();
  }

  // epilogue: O = acc / l (bf16, RNE); LSE = (m + log2 l) ln 2
  const float l_tot = l_run + swap_halves(l_run);
  const float inv = l_tot > 0.f ? 1.f / l_tot : 0.f;
  const int row = qw0 + n;
  if (row < p.Nq) {
    uint16_t* op = p.o + ((int64_t)b * p.Nq + row) * q_row + (int64_t)h * D;
#pragma unroll
    for (int db = 0; db < T::NDB; ++db)
#pragma unroll
      for (int r4 = 0; r4 < 4; ++r4) {
        const int d = db * 32 + r4 * 8 + g * 4;
        u32x2 w;
        w[0] = pack_bf16x2(acc[db][r4 * 4 + 0] * inv, acc[db][r4 * 4 + 1] * inv);
        w[1] = pack_bf16x2(acc[db][r4 * 4 + 2] * inv, acc[db][r4 * 4 + 3] * inv);
        *reinterpret_cast<u32x2*>(op + d) = w;
      }
    if (p.lse != nullptr && g == 0)
      p.lse[((int64_t)b * p.Hq + h) * p.Nq + row] =
          l_tot > 0.f ? (m_run + fast_log2(l_tot)) * kLn2 : kNegInf;
  }
}

}  // namespace

long long fwd_bf16_grid(int B, int Hq, int Nq) {
  return (long long)B * Hq * ((Nq + kBM - 1) / kBM);
}

hipError_t launch_fwd_bf16(const FwdArgs& a, hipStream_t stream) {
  Params p;
  p.q = static_cast<const uint16_t*>(a.q);
  p.k = static_cast<const uint16_t*>(a.k);
  p.v = static_cast<const uint16_t*>(a.v);
  p.o = static_cast<uint16_t*>(a.out);
  p.lse = a.lse;
  p.Hq = a.Hq;
  p.Hkv = a.Hkv;
  p.group = a.Hq / a.Hkv;
  p.Nq = a.Nq;
  p.Nk = a.Nk;
  p.causal = a.causal;
  p.window = a.window;
  p.n_qtiles = (a.Nq + kBM - 1) / kBM;
  p.total = (int)fwd_bf16_grid(a.B, a.Hq, a.Nq);
  p.sl2 = a.scale * kLog2e;
  if (p.total == 0) return hipSuccess;
  const dim3 grid(p.total), block(kThreads);
  if (a.d == 128)
    hipLaunchKernelGGL(fwd_bf16_kernel<128>, grid, block, 0, stream, p);
  else
    hipLaunchKernelGGL(fwd_bf16_kernel<64>, grid, block, 0, stream, p);
  return hipGetLastError();
}

}  // namespace attn
