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
//     registers (converted to bf16, round-to-nearest-even; the row sum is
//     taken over the float32 values, so LSE is exact to fp32), A = V^T read from
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
constexpr float kLazy = 8.0f;  // rescale only when a row max grows by more than 2^8

typedef short s16x4 __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) s16x4 lds_s16x4;

template <int D>
struct Tile {
  static constexpr int BN = 64;                      // keys per tile
  static constexpr int NKB = BN / 32;                // 32-key blocks of S^T
  static constexpr int NDB = D / 32;                 // 32-feature blocks of O^T
  static constexpr int KC = D / 16;                  // k-chunks of K Q^T
  static constexpr int VC = BN / 16;                 // k-chunks of V^T P^T
  // Row strides in LDS (bf16 elements).  K rows are read 16 bytes per lane
  // down 16 consecutive rows: a stride of 16*odd bytes spreads them over all
  // banks.  V rows are read with the transposing LDS load, 4 rows x 64 bytes
  // per half wave: a stride of 64 or 192 bytes past a multiple of 256 does.
  static constexpr int KSTRIDE = D + 8;
  static constexpr int VSTRIDE = D + 32;
  static constexpr int K_ELEMS = BN * KSTRIDE;
  static constexpr int V_ELEMS = BN * VSTRIDE;
  static constexpr int STAGE = K_ELEMS + V_ELEMS;
  static constexpr int CHUNKS = BN * D / 8 / kThreads;  // 16-byte pieces per thread, each of K and V
  static_assert(CHUNKS * kThreads * 8 == BN * D, "staging must cover the tile");
  static_assert((VSTRIDE * 2) % 128 == 64, "V rows must fall 64 bytes apart modulo 128");
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

// POS_SCALE: scale > 0, so the row maximum of scale*s is scale * max(s) and the
// scaling folds into the exponent's FMA.  Otherwise every score is scaled first.
template <int D, bool POS_SCALE>
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
    const int row = min(qw0 + n, p.Nq - 1);  // rows past the end compute garbage, never stored
    const uint16_t* qp = p.q + ((int64_t)b * p.Nq + row) * q_row + (int64_t)h * D + g * 8;
#pragma unroll
    for (int c = 0; c < T::KC; ++c) qf[c] = *reinterpret_cast<const bf16x8*>(qp + c * 16);
  }

  const int64_t kv_row = (int64_t)p.Hkv * D;
  const uint16_t* kbase = p.k + (int64_t)b * p.Nk * kv_row + (int64_t)hk * D;
  const uint16_t* vbase = p.v + (int64_t)b * p.Nk * kv_row + (int64_t)hk * D;

  // Staging: piece c of this thread is row (tid + c*256) / (D/8) of the tile,
  // 16-byte column (tid % (D/8)).  Rows past the last key re-read the last
  // key: their scores are masked and their probabilities are exactly zero, so
  // a finite duplicate contributes nothing and no load needs a branch.
  u32x4 kreg[T::CHUNKS], vreg[T::CHUNKS];
  const int col8 = tid % (D / 8);
  const int row0 = tid / (D / 8);
  constexpr int kRowStep = kThreads / (D / 8);
  auto load_tile = [&](int t) {
    const int j0 = t * T::BN;
#pragma unroll
    for (int c = 0; c < T::CHUNKS; ++c) {
      const int j = min(j0 + row0 + c * kRowStep, p.Nk - 1);
      const int64_t off = (int64_t)j * kv_row + col8 * 8;
      kreg[c] = *reinterpret_cast<const u32x4*>(kbase + off);
      vreg[c] = *reinterpret_cast<const u32x4*>(vbase + off);
    }
  };
  auto store_tile = [&](int buf) {
    uint16_t* ks = smem + buf * T::STAGE;
    uint16_t* vs = ks + T::K_ELEMS;
#pragma unroll
    for (int c = 0; c < T::CHUNKS; ++c) {
      const int row = row0 + c * kRowStep;
      *reinterpret_cast<u32x4*>(ks + row * T::KSTRIDE + col8 * 8) = kreg[c];
      *reinterpret_cast<u32x4*>(vs + row * T::VSTRIDE + col8 * 8) = vreg[c];
    }
  };

  // Transposed V reads: for MFMA k-chunk kc and feature block db, lane
  // (group G = lane/16, s = lane%16) points at key kc*16 + (G/2)*4 + s/4
  // (+8 for the second read) and features db*32 + 16*(G%2) + 4*(s%4).  The
  // hardware hands lane 4r+c of each 16-lane group the 4 keys of source lanes
  // r, r+4, r+8, r+12 at feature 4r+c, which is V^T in the operand layout, with
  // lane group g holding keys {g*4..g*4+3, 8+g*4..8+g*4+3} of the chunk.
  const int G16 = lane >> 4, s16 = lane & 15;
  const int vt_key = (G16 >> 1) * 4 + (s16 >> 2);
  const int vt_col = 16 * (G16 & 1) + 4 * (s16 & 3);

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

      if (!POS_SCALE) {
#pragma unroll
        for (int kb = 0; kb < T::NKB; ++kb)
#pragma unroll
          for (int r = 0; r < 16; ++r) st[kb][r] *= p.sl2;
      }
      // mask only tiles that cut the causal/window band or the key tail
      const bool need_mask = (j0 + T::BN > p.Nk) ||
                             (p.causal && j0 + T::BN - 1 > qw0 + delta) ||
                             (p.window > 0 && qw0 + kRowsPerWave - 1 + delta - j0 >= p.window);
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

      // online softmax with a lazily raised maximum: the stored max only moves
      // when some row's max exceeds it by more than 2^8, so most tiles skip
      // the accumulator rescale; probabilities stay <= 2^8, and the final
      // division uses the sum taken at the same max, so the result is exact.
      float mx = kNegInf;
#pragma unroll
      for (int kb = 0; kb < T::NKB; ++kb)
#pragma unroll
        for (int r = 0; r < 16; ++r) mx = fmaxf(mx, st[kb][r]);
      mx = fmaxf(mx, swap_halves(mx));
      if (POS_SCALE) mx *= p.sl2;
      if (__builtin_amdgcn_ballot_w64(mx > m_run + kLazy) != 0) {
        const float m_new = fmaxf(m_run, mx);
        const float alpha = (m_new == kNegInf) ? 1.f : fast_exp2(m_run - m_new);
        l_run *= alpha;
#pragma unroll
        for (int db = 0; db < T::NDB; ++db)
#pragma unroll
          for (int r = 0; r < 16; ++r) acc[db][r] *= alpha;
        m_run = m_new;
      }
      const float m_use = (m_run == kNegInf) ? 0.f : m_run;  // row with nothing visible yet

      uint32_t pk[T::NKB][8];
      float rs = 0.f;
#pragma unroll
      for (int kb = 0; kb < T::NKB; ++kb)
#pragma unroll
        for (int i = 0; i < 8; ++i) {
          float p0, p1;
          if (POS_SCALE) {
            p0 = fast_exp2(fmaf(st[kb][2 * i], p.sl2, -m_use));
            p1 = fast_exp2(fmaf(st[kb][2 * i + 1], p.sl2, -m_use));
          } else {
            p0 = fast_exp2(st[kb][2 * i] - m_use);
            p1 = fast_exp2(st[kb][2 * i + 1] - m_use);
          }
          pk[kb][i] = pack_bf16x2(p0, p1);
          rs += p0 + p1;  // float32 sum: the LSE must reproduce exp(S - LSE) to fp32
        }
      l_run += rs;

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
        const uint16_t* vrow = vs + (kc * 16 + vt_key) * T::VSTRIDE + vt_col;
#pragma unroll
        for (int db = 0; db < T::NDB; ++db) {
          const s16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
              (lds_s16x4*)(vrow + db * 32));
          const s16x4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
              (lds_s16x4*)(vrow + 8 * T::VSTRIDE + db * 32));
          const bf16x8 vf =
              __builtin_bit_cast(bf16x8, __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7));
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
  const bool pos = a.scale > 0.f;
  if (a.d == 128) {
    if (pos)
      hipLaunchKernelGGL((fwd_bf16_kernel<128, true>), grid, block, 0, stream, p);
    else
      hipLaunchKernelGGL((fwd_bf16_kernel<128, false>), grid, block, 0, stream, p);
  } else {
    if (pos)
      hipLaunchKernelGGL((fwd_bf16_kernel<64, true>), grid, block, 0, stream, p);
    else
      hipLaunchKernelGGL((fwd_bf16_kernel<64, false>), grid, block, 0, stream, p);
  }
  return hipGetLastError();
}

}  // namespace attn
