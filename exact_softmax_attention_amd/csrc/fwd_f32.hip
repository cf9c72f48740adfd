// Tiled, fused forward for float32 Q/K/V on gfx950: the same loop as the
// bf16 kernel ("Attention Is O(n^2)", section "FlashAttention - Same FLOPs,
// Linear Memory"), with every product and sum in float32.
//
// Both contractions use v_mfma_f32_32x32x2_f32, which multiplies float32
// operands and accumulates in float32 (no reduced-precision input format).
//   * S^T = K Q^T: lane (n, g) supplies K[key n][d] and Q[row n][d] for
//     features d in its half g of the head dimension, one per instruction.
//   * O^T = V^T P^T: the probabilities stay float32 in the accumulator
//     registers; the k index of each instruction is one key, and lane (n, g)
//     supplies V[that key][feature n] (a row-major LDS read, conflict-free)
//     and its own P value for that key.
// 4 waves x 32 query rows per work group, 32 keys per tile, two LDS buffers.
#include "device_common.h"
#include "launch.h"

namespace attn {
namespace {

constexpr int kWaves = 4;
constexpr int kRowsPerWave = 32;
constexpr int kBM = kWaves * kRowsPerWave;
constexpr int kThreads = kWaves * 64;
constexpr int kBN = 32;

template <int D>
struct TileF {
  static constexpr int NDB = D / 32;
  static constexpr int HALF = D / 2;             // features per lane group
  static constexpr int KSTRIDE = D + 4;          // floats per K row in LDS
  static constexpr int K_ELEMS = kBN * KSTRIDE;
  static constexpr int V_ELEMS = kBN * D;
  static constexpr int STAGE = K_ELEMS + V_ELEMS;
  static constexpr int CHUNKS = kBN * D / 4 / kThreads;  // 16-byte pieces per thread
  static_assert(CHUNKS * kThreads * 4 == kBN * D, "staging must cover the tile");
};

struct Params {
  const float* q;
  const float* k;
  const float* v;
  float* o;
  float* lse;
  int Hq, Hkv, group, Nq, Nk, causal, window, n_qtiles, total;
  float sl2;
};

template <int D>
__global__ __launch_bounds__(kThreads, 2) void fwd_f32_kernel(const Params p) {
  using T = TileF<D>;
  __shared__ __attribute__((aligned(16))) float smem[2 * T::STAGE];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int n = lane & 31;
  const int g = lane >> 5;

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
  const int t_begin = kv_begin / kBN;
  const int t_end = kv_end > kv_begin ? (kv_end + kBN - 1) / kBN : t_begin;

  const int64_t q_row = (int64_t)p.Hq * D;
  float qf[T::HALF];
  {
    const int row = qw0 + n;
    if (row < p.Nq) {
      const float* qp = p.q + ((int64_t)b * p.Nq + row) * q_row + (int64_t)h * D + g * T::HALF;
#pragma unroll
      for (int c = 0; c < T::HALF; c += 4) {
        const f32x4 x = *reinterpret_cast<const f32x4*>(qp + c);
        qf[c] = x[0];
        qf[c + 1] = x[1];
        qf[c + 2] = x[2];
        qf[c + 3] = x[3];
      }
    } else {
#pragma unroll
      for (int c = 0; c < T::HALF; ++c) qf[c] = 0.f;
    }
  }

  const int64_t kv_row = (int64_t)p.Hkv * D;
  const float* kbase = p.k + (int64_t)b * p.Nk * kv_row + (int64_t)hk * D;
  const float* vbase = p.v + (int64_t)b * p.Nk * kv_row + (int64_t)hk * D;

  f32x4 kreg[T::CHUNKS], vreg[T::CHUNKS];
  auto load_tile = [&](int t) {
    const int j0 = t * kBN;
#pragma unroll
    for (int c = 0; c < T::CHUNKS; ++c) {
      const int cid = tid + c * kThreads;
      const int row = cid / (D / 4);
      const int col = cid % (D / 4);
      const int j = j0 + row;
      if (j < p.Nk) {
        kreg[c] = *reinterpret_cast<const f32x4*>(kbase + (int64_t)j * kv_row + col * 4);
        vreg[c] = *reinterpret_cast<const f32x4*>(vbase + (int64_t)j * kv_row + col * 4);
      } else {
        kreg[c] = f32x4{};
        vreg[c] = f32x4{};
      }
    }
  };
  auto store_tile = [&](int buf) {
    float* ks = smem + buf * T::STAGE;
    float* vs = ks + T::K_ELEMS;
#pragma unroll
    for (int c = 0; c < T::CHUNKS; ++c) {
      const int cid = tid + c * kThreads;
      const int row = cid / (D / 4);
      const int col = cid % (D / 4);
      *reinterpret_cast<f32x4*>(ks + row * T::KSTRIDE + col * 4) = kreg[c];
      *reinterpret_cast<f32x4*>(vs + row * D + col * 4) = vreg[c];
    }
  };

  float m_run = kNegInf;
  float l_run = 0.f;
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
    const int j0 = t * kBN;

    bool skip = qw0 >= p.Nq;
    if (p.causal && j0 > qw0 + kRowsPerWave - 1 + delta) skip = true;
    if (p.window > 0 && j0 + kBN - 1 < qw0 + delta - p.window + 1) skip = true;

    if (!skip) {
      const float* ks = smem + buf * T::STAGE;
      const float* vs = ks + T::K_ELEMS;

      f32x16 st = f32x16{};
      const float* krow = ks + n * T::KSTRIDE + g * T::HALF;
#pragma unroll
      for (int c = 0; c < T::HALF; c += 4) {
        const f32x4 kf = *reinterpret_cast<const f32x4*>(krow + c);
        st = __builtin_amdgcn_mfma_f32_32x32x2f32(kf[0], qf[c], st, 0, 0, 0);
        st = __builtin_amdgcn_mfma_f32_32x32x2f32(kf[1], qf[c + 1], st, 0, 0, 0);
        st = __builtin_amdgcn_mfma_f32_32x32x2f32(kf[2], qf[c + 2], st, 0, 0, 0);
        st = __builtin_amdgcn_mfma_f32_32x32x2f32(kf[3], qf[c + 3], st, 0, 0, 0);
      }

      const bool need_mask = (j0 + kBN > p.Nk) ||
                             (p.causal && j0 + kBN - 1 > qw0 + delta) ||
                             (p.window > 0 && qw0 + kRowsPerWave - 1 + delta - j0 >= p.window);
#pragma unroll
      for (int r = 0; r < 16; ++r) st[r] *= p.sl2;
      if (need_mask) {
        const int pos = qw0 + n + delta;
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const int key = j0 + (r >> 2) * 8 + g * 4 + (r & 3);
          bool vis = key < p.Nk;
          if (p.causal) vis = vis && key <= pos;
          if (p.window > 0) vis = vis && (pos - key) < p.window;
          if (!vis) st[r] = kNegInf;
        }
      }

      float mx = kNegInf;
#pragma unroll
      for (int r = 0; r < 16; ++r) mx = fmaxf(mx, st[r]);
      mx = fmaxf(mx, swap_halves(mx));
      const float m_new = fmaxf(m_run, mx);
      const float m_use = (m_new == kNegInf) ? 0.f : m_new;
      const float alpha = fast_exp2(m_run - m_use);
      m_run = m_new;

      float rs = 0.f;
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        st[r] = fast_exp2(st[r] - m_use);
        rs += st[r];
      }
      l_run = l_run * alpha + rs;
#pragma unroll
      for (int db = 0; db < T::NDB; ++db)
#pragma unroll
        for (int r = 0; r < 16; ++r) acc[db][r] *= alpha;

#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int key = (r >> 2) * 8 + g * 4 + (r & 3);
#pragma unroll
        for (int db = 0; db < T::NDB; ++db)
          acc[db] = __builtin_amdgcn_mfma_f32_32x32x2f32(vs[key * D + db * 32 + n], st[r],
                                                         acc[db], 0, 0, 0);
      }
    }

    if (has_next) store_tile(buf ^ 1);
    __syncthreads();
  }

  const float l_tot = l_run + swap_halves(l_run);
  const float inv = l_tot > 0.f ? 1.f / l_tot : 0.f;
  const int row = qw0 + n;
  if (row < p.Nq) {
    float* op = p.o + ((int64_t)b * p.Nq + row) * q_row + (int64_t)h * D;
#pragma unroll
    for (int db = 0; db < T::NDB; ++db)
#pragma unroll
      for (int r4 = 0; r4 < 4; ++r4) {
        const int d = db * 32 + r4 * 8 + g * 4;
        f32x4 w;
        w[0] = acc[db][r4 * 4 + 0] * inv;
        w[1] = acc[db][r4 * 4 + 1] * inv;
        w[2] = acc[db][r4 * 4 + 2] * inv;
        w[3] = acc[db][r4 * 4 + 3] * inv;
        *reinterpret_cast<f32x4*>(op + d) = w;
      }
    if (p.lse != nullptr && g == 0)
      p.lse[((int64_t)b * p.Hq + h) * p.Nq + row] =
          l_tot > 0.f ? (m_run + log2f(l_tot)) * kLn2 : kNegInf;
  }
}

}  // namespace

long long fwd_f32_grid(int B, int Hq, int Nq) {
  return (long long)B * Hq * ((Nq + kBM - 1) / kBM);
}

hipError_t launch_fwd_f32(const FwdArgs& a, hipStream_t stream) {
  Params p;
  p.q = static_cast<const float*>(a.q);
  p.k = static_cast<const float*>(a.k);
  p.v = static_cast<const float*>(a.v);
  p.o = static_cast<float*>(a.out);
  p.lse = a.lse;
  p.Hq = a.Hq;
  p.Hkv = a.Hkv;
  p.group = a.Hq / a.Hkv;
  p.Nq = a.Nq;
  p.Nk = a.Nk;
  p.causal = a.causal;
  p.window = a.window;
  p.n_qtiles = (a.Nq + kBM - 1) / kBM;
  p.total = (int)fwd_f32_grid(a.B, a.Hq, a.Nq);
  p.sl2 = a.scale * kLog2e;
  if (p.total == 0) return hipSuccess;
  const dim3 grid(p.total), block(kThreads);
  if (a.d == 128)
    hipLaunchKernelGGL(fwd_f32_kernel<128>, grid, block, 0, stream, p);
  else
    hipLaunchKernelGGL(fwd_f32_kernel<64>, grid, block, 0, stream, p);
  return hipGetLastError();
}

}  // namespace attn
