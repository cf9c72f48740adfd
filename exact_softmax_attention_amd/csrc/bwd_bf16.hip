// Backward pass of exact softmax attention for bf16 Q/K/V on gfx950.
//
// Method: the backward pass recomputes the local probabilities from the
// statistics the forward saved instead of storing the attention matrix
// ("Ch. 3: MHA Limitations, MQA, GQA, and FlashAttention", section 3.5; the
// float32 log-sum-exp of "Attention Is O(n^2): FlashAttention vs Linear
// Attention", section "FlashAttention - Same FLOPs, Linear Memory").  With
// P = exp(scale * Q K^T - LSE) over the visible keys, the gradients of
// L = sum(dO * O) are
//     dV = P^T dO,  dP = dO V^T,  D_i = sum_c dO_ic O_ic,
//     dS = P * (dP - D),  dQ = scale * dS K,  dK = scale * dS^T Q,
// and a KV head shared by G query heads sums their dK and dV.
//
// Three kernels, no atomics (the results do not depend on scheduling):
//   bwd_prep   D = rowsum(dO * O) and LSE * log2(e) per (b, h, row), into the
//              workspace (a row with LSE = -inf, which sees no key, gets
//              +inf, so that all its probabilities come out 0).
//   bwd_dkdv   one work group per (128-key tile, KV head, batch); wave w owns
//              32 keys, holding them as the B operand of
//              v_mfma_f32_32x32x16_bf16 (lane l: key l % 32).  It walks the G
//              query heads and their 32-row query blocks that see the tile:
//                S  = Q K^T     A = Q rows from LDS, B = K (registers)
//                dP = dO V^T    A = dO rows from LDS, B = V (registers)
//              (lane l: key l % 32, 16 query rows), then P, dS, and
//                dV^T += dO^T P   A = dO^T from the LDS transposing load
//                dK^T += Q^T dS   A = Q^T likewise
//              with P and dS converted to bf16 (round to nearest even) as the
//              B operands straight from the score registers: the MFMA k index
//              runs over the query rows in the same permuted order on both
//              operands.
//   bwd_dq     one work group per 128-row query tile of one head; wave w owns
//              32 rows, holding Q and dO as B operands (lane l: row l % 32):
//                S^T = K Q^T,  dP^T = V dO^T   A = K, V rows from LDS
//                dQ^T += K^T dS^T              A = K^T from the transposing load
//              so P, D and the log-sum-exp are one value per lane.
// Tiles go through registers into LDS (double-buffered: the next tile's
// global loads are in flight while the current one is computed).  Rows are
// padded to a pitch of 2D + 16 bytes, which keeps both the row reads and the
// transposing reads of the same tile free of most bank conflicts.
#include <type_traits>

#include "device_common.h"
#include "launch.h"

namespace attn {
namespace {

typedef short s16x4 __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) s16x4 lds_s16x4;
typedef __attribute__((address_space(3))) uint8_t lds_u8;

constexpr int kBwdWaves = 4;
constexpr int kBwdThreads = kBwdWaves * 64;
constexpr int kBlk = 32;  // MFMA block: 32 keys x 32 query rows
constexpr int kAhead = 3; // tiles whose global loads are in flight (in registers)

// f(integral_constant<0>) .. f(integral_constant<N-1>) while f returns true;
// the index is a compile-time constant, so register sets can be chosen by it.
template <int I, int N, typename F>
__device__ __forceinline__ bool unroll_while(F&& f) {
  if constexpr (I < N) {
    if (!f(std::integral_constant<int, I>{})) return false;
    return unroll_while<I + 1, N>(f);
  }
  return true;
}

struct BwdParams {
  const uint16_t* q;
  const uint16_t* k;
  const uint16_t* v;
  const uint16_t* o;
  const uint16_t* dout;
  const float* lse;
  uint16_t* dq;
  uint16_t* dk;
  uint16_t* dv;
  float* dsum;   // [B, Hq, Nq] ([Hq, total_q] packed): D = rowsum(dO * O)
  float* lse2;   // same layout: LSE * log2(e), +inf for a row without keys
  int B, Hq, Hkv, group, Nq, Nk, causal, window;
  float scale, sl2;
  // packed sequences: sequence s owns query rows [cu_q[s], cu_q[s+1]) and key
  // rows [cu_k[s], cu_k[s+1]); LSE, D and lse2 are [Hq, total_q]
  const int* cu_q;
  const int* cu_k;
  int n_seqs, total_q, total_k;
};

// The sequence and 128-row tile of a work group.  Dense: sequence blockIdx.z,
// tile blockIdx.x.  Packed: blockIdx.x is a slot of the packed axis (queries
// or keys, `cu` and `total`), the slots of sequence s starting at
// cu[s] / 128 + s; tile < 0 for a slot past the sequence's tiles.
struct SeqTile {
  int b, tile, Nq, Nk;
  int64_t q0, k0;  // first query and key row of the sequence
  __device__ int64_t stat(const BwdParams& p, int h, bool packed) const {  // LSE index of row 0
    return packed ? (int64_t)h * p.total_q + q0 : ((int64_t)b * p.Hq + h) * Nq;
  }
};

template <bool VARLEN>
__device__ __forceinline__ SeqTile seq_tile(const BwdParams& p, const int* cu, int total,
                                            int lane) {
  SeqTile t;
  if constexpr (VARLEN) {
    constexpr int TILE = kBwdWaves * kBlk;
    const int slot = blockIdx.x;
    t.b = find_seq<TILE>(cu, p.n_seqs, total, slot, lane);
    const int q0 = clampi(p.cu_q[t.b], 0, p.total_q);
    const int k0 = clampi(p.cu_k[t.b], 0, p.total_k);
    t.Nq = clampi(p.cu_q[t.b + 1], q0, p.total_q) - q0;
    t.Nk = clampi(p.cu_k[t.b + 1], k0, p.total_k) - k0;
    t.q0 = q0;
    t.k0 = k0;
    const int a0 = clampi(cu[t.b], 0, total);
    const int len = cu == p.cu_q ? t.Nq : t.Nk;
    const int off = slot - (a0 / TILE + t.b);
    t.tile = (off >= 0 && off * TILE < len) ? off : -1;
  } else {
    t.b = blockIdx.z;
    t.tile = blockIdx.x;
    t.Nq = p.Nq;
    t.Nk = p.Nk;
    t.q0 = (int64_t)t.b * p.Nq;
    t.k0 = (int64_t)t.b * p.Nk;
  }
  return t;
}

template <int D>
struct BT {
  static constexpr int KC = D / 16;            // k-chunks over the head dimension
  static constexpr int NDB = D / 32;           // 32-feature blocks of dK^T, dV^T, dQ^T
  static constexpr int PITCH = 2 * D + 16;     // LDS bytes per staged row
  static constexpr int ROWB = 2 * D;           // global bytes per row
  static constexpr int PIECES = ROWB / 16;     // 16-byte pieces per row
};

// ---------------------------------------------------------------------------
// Shared tile helpers.

// Stage ROWS rows (16-byte pieces) of a [N, H, D] tensor starting at row r0
// into registers: piece p of the block = row p / PIECES, piece p % PIECES.
// The loads are buffer loads whose range ends with row n_rows - 1, so rows at
// or past n_rows read as zero; each thread's byte offsets within the block
// are fixed (StageOff) and only the scalar base moves from step to step.
template <int D, int ROWS>
struct StageOff {
  static constexpr int NP = ROWS * BT<D>::PIECES / kBwdThreads;  // pieces per thread
  static_assert(NP * kBwdThreads == ROWS * BT<D>::PIECES, "whole pieces per thread");
  int off[NP];
  __device__ __forceinline__ StageOff(int64_t row_stride, int tid) {
#pragma unroll
    for (int i = 0; i < NP; ++i) {
      const int p = tid + i * kBwdThreads;
      off[i] = (int)((p / BT<D>::PIECES) * row_stride * 2) + (p % BT<D>::PIECES) * 16;
    }
  }
};

template <int D, int ROWS>
struct Stage {
  static constexpr int NP = StageOff<D, ROWS>::NP;
  u32x4 r[NP];
  __device__ __forceinline__ void load(const uint16_t* base, int64_t row_stride, int r0, int n_rows,
                                       const StageOff<D, ROWS>& so) {
    const int real = min(ROWS, n_rows - r0);  // rows of the block that exist (>= 1)
    const int bytes = (int)((real - 1) * row_stride * 2) + 2 * D;
    const __amdgpu_buffer_rsrc_t rs = __builtin_amdgcn_make_buffer_rsrc(
        const_cast<uint16_t*>(base + (int64_t)r0 * row_stride), (short)0, bytes, 0x00020000);
#pragma unroll
    for (int i = 0; i < NP; ++i)
      r[i] = __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(rs, so.off[i], 0, 0));
  }
  __device__ __forceinline__ void store(lds_u8* lds, uint32_t off, int tid) const {
#pragma unroll
    for (int i = 0; i < NP; ++i) {
      const int p = tid + i * kBwdThreads;
      const int row = p / BT<D>::PIECES, pc = p % BT<D>::PIECES;
      *reinterpret_cast<__attribute__((address_space(3))) u32x4*>(lds + off + row * BT<D>::PITCH + pc * 16) = r[i];
    }
  }
};

// A operand (rows x k) of a 32x32x16 MFMA from a staged tile: lane l reads row
// row0 + l % 32, features 16c + 8 (l / 32) .. +7.
template <int D>
__device__ __forceinline__ bf16x8 row_frag(const lds_u8* lds, uint32_t off, int lane, int c) {
  const uint32_t a = off + (lane & 31) * BT<D>::PITCH + (16 * c + 8 * (lane >> 5)) * 2;
  return *reinterpret_cast<const __attribute__((address_space(3))) bf16x8*>(lds + a);
}

// A operand (features x rows) = the tile transposed, for feature block db and
// row chunk kc (16 rows): the transposing load hands lane 4r+c of each 16-lane
// group the 4 rows of source lanes r, r+4, r+8, r+12 at feature 4r+c, so lane
// l gets feature 32 db + l % 32 and rows {4g..4g+3, 8+4g..8+4g+3} + 16 kc,
// g = l / 32: the order in which the 32x32 accumulator layout holds rows.
template <int D>
__device__ __forceinline__ bf16x8 tr_frag(const lds_u8* lds, uint32_t off, int lane, int db, int kc) {
  const int G16 = lane >> 4, s16 = lane & 15;
  const int row = kc * 16 + (G16 >> 1) * 4 + (s16 >> 2);
  const int feat = db * 32 + 16 * (G16 & 1) + 4 * (s16 & 3);
  const uint32_t a = off + row * BT<D>::PITCH + feat * 2;
  const s16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4*)(lds + a));
  const s16x4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4*)(lds + a + 8 * BT<D>::PITCH));
  return __builtin_bit_cast(bf16x8, __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7));
}

// ---------------------------------------------------------------------------
// D and LSE * log2(e) per row.

template <int D, bool VARLEN>
__global__ __launch_bounds__(256) void bwd_prep_kernel(const BwdParams p) {
  constexpr int LPR = D / 8;          // lanes per row (16 bytes each)
  constexpr int RPB = 256 / LPR;      // rows per block step
  const int tid = threadIdx.x;
  const int sub = tid % LPR;
  // rows in [B, Nq, Hq] (packed: [total_q, Hq]) order
  const int64_t rows = VARLEN ? (int64_t)p.total_q * p.Hq : (int64_t)p.B * p.Nq * p.Hq;
  for (int64_t r = (int64_t)blockIdx.x * RPB + tid / LPR; r < rows; r += (int64_t)gridDim.x * RPB) {
    const u32x4 a = *reinterpret_cast<const u32x4*>(p.dout + r * D + sub * 8);
    const u32x4 b = *reinterpret_cast<const u32x4*>(p.o + r * D + sub * 8);
    float s = 0.f;
#pragma unroll
    for (int i = 0; i < 4; ++i)
      s += bf16lo_to_f32(a[i]) * bf16lo_to_f32(b[i]) + bf16hi_to_f32(a[i]) * bf16hi_to_f32(b[i]);
#pragma unroll
    for (int o = LPR / 2; o >= 1; o >>= 1) s += __shfl_xor(s, o, LPR);
    if (sub == 0) {
      const int h = (int)(r % p.Hq);
      const int64_t bi = r / p.Hq;
      int64_t o;
      if constexpr (VARLEN) {
        o = (int64_t)h * p.total_q + bi;
      } else {
        const int i = (int)(bi % p.Nq);
        const int b = (int)(bi / p.Nq);
        o = ((int64_t)b * p.Hq + h) * p.Nq + i;
      }
      const float l = p.lse[o];
      p.dsum[o] = s;
      p.lse2[o] = l == kNegInf ? __builtin_inff() : l * kLog2e;
    }
  }
}

// ---------------------------------------------------------------------------
// dK, dV.

template <int D, bool VARLEN>
__global__ __launch_bounds__(kBwdThreads) void bwd_dkdv_kernel(const BwdParams p) {
  using T = BT<D>;
  constexpr int QTILE = T::PITCH * kBlk;  // bytes of one staged 32-row tile
  // [buffer][Q, dO] tiles, then [buffer][lse2, D] (32 floats each)
  __shared__ __attribute__((aligned(16))) uint8_t smem[2 * 2 * QTILE + 2 * 2 * kBlk * 4];
  lds_u8* const lds = (lds_u8*)smem;
  const uint32_t stat0 = 4 * QTILE;

  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const SeqTile sq = seq_tile<VARLEN>(p, p.cu_k, p.total_k, lane);
  if (sq.tile < 0) return;  // a schedule slot past the sequence (whole group)
  const int Nq = sq.Nq, Nk = sq.Nk;
  const int kt = sq.tile, hk = blockIdx.y;
  const int k0 = kt * kBwdWaves * kBlk;          // first key of the tile
  const int kw0 = k0 + wave * kBlk;              // first key of this wave
  const int key = kw0 + (lane & 31);             // this lane's key (column)
  const int g = lane >> 5;
  const int delta = Nk - Nq;
  const int64_t kv_row = (int64_t)p.Hkv * D;
  const int64_t q_row = (int64_t)p.Hq * D;

  // K and V of the lane's key as B operands (features 16c + 8g .. +7)
  bf16x8 kb[T::KC], vb[T::KC];
  {
    const int64_t off = (sq.k0 + key) * kv_row + (int64_t)hk * D + 8 * g;
#pragma unroll
    for (int c = 0; c < T::KC; ++c) {
      u32x4 x = {0u, 0u, 0u, 0u}, y = {0u, 0u, 0u, 0u};
      if (key < Nk) {
        x = *reinterpret_cast<const u32x4*>(p.k + off + 16 * c);
        y = *reinterpret_cast<const u32x4*>(p.v + off + 16 * c);
      }
      kb[c] = __builtin_bit_cast(bf16x8, x);
      vb[c] = __builtin_bit_cast(bf16x8, y);
    }
  }
  f32x16 dkt[T::NDB], dvt[T::NDB];
#pragma unroll
  for (int db = 0; db < T::NDB; ++db) dkt[db] = dvt[db] = f32x16{};

  // query rows that see some key of the tile: [qlo, qhi)
  const int klast = min(Nk, k0 + kBwdWaves * kBlk) - 1;
  int qlo = 0, qhi = Nq;
  if (p.causal) qlo = max(0, k0 - delta);
  if (p.window > 0) qhi = min(Nq, klast - delta + p.window);
  const int nblk = qhi > qlo ? (qhi - (qlo & ~(kBlk - 1)) + kBlk - 1) / kBlk : 0;
  const int q_first = qlo & ~(kBlk - 1);
  const int steps = nblk * p.group;  // (head, block) pairs, head-major

  // step t's tiles travel in register set t % kAhead: loaded kAhead steps
  // before they are computed, stored to LDS buffer t % 2 one step before
  struct Set {
    Stage<D, kBlk> q, o;
    float l2, d;  // lse2 and D of row tid (tid < 32)
  };
  Set sets[kAhead];
  const StageOff<D, kBlk> so(q_row, tid);
  auto fetch = [&](Set& st, int s) __attribute__((always_inline)) {
    if (s >= steps) return;
    const int h = hk * p.group + s / nblk;
    const int i0 = q_first + (s % nblk) * kBlk;
    const uint16_t* qb = p.q + sq.q0 * q_row + (int64_t)h * D;
    const uint16_t* ob = p.dout + sq.q0 * q_row + (int64_t)h * D;
    st.q.load(qb, q_row, i0, Nq, so);
    st.o.load(ob, q_row, i0, Nq, so);
    if (tid < kBlk) {
      const int i = i0 + tid;
      const int64_t o = sq.stat(p, h, VARLEN) + i;
      st.l2 = i < Nq ? p.lse2[o] : __builtin_inff();
      st.d = i < Nq ? p.dsum[o] : 0.f;
    }
  };
  auto stash = [&](const Set& st, int buf) __attribute__((always_inline)) {
    st.q.store(lds, (2 * buf) * QTILE, tid);
    st.o.store(lds, (2 * buf + 1) * QTILE, tid);
    if (tid < kBlk) {
      *reinterpret_cast<__attribute__((address_space(3))) float*>(lds + stat0 + (2 * buf) * kBlk * 4 + tid * 4) = st.l2;
      *reinterpret_cast<__attribute__((address_space(3))) float*>(lds + stat0 + (2 * buf + 1) * kBlk * 4 + tid * 4) = st.d;
    }
  };

  unroll_while<0, kAhead>([&](auto J) { fetch(sets[J], J); return true; });
  if (steps > 0) {
    stash(sets[0], 0);
    fetch(sets[0], kAhead);
  }
  __syncthreads();
  for (int s0 = 0; s0 < steps; s0 += kAhead) {
   const bool more = unroll_while<0, kAhead>([&](auto U) __attribute__((always_inline)) {
    constexpr int u = decltype(U)::value;
    const int s = s0 + u;
    if (s >= steps) return false;
    const int buf = s & 1;
    const int i0 = q_first + (s % nblk) * kBlk;
    const uint32_t qoff = (2 * buf) * QTILE, ooff = (2 * buf + 1) * QTILE;
    const uint32_t loff = stat0 + (2 * buf) * kBlk * 4, doff = stat0 + (2 * buf + 1) * kBlk * 4;
    // does this wave's 32 x 32 block hold any visible pair, and does it need a mask?
    bool any = kw0 < Nk;
    if (p.causal && kw0 > i0 + kBlk - 1 + delta) any = false;
    if (p.window > 0 && i0 + delta - (kw0 + kBlk - 1) >= p.window) any = false;
    const bool full = (!p.causal || kw0 + kBlk - 1 <= i0 + delta) &&
                      (p.window <= 0 || i0 + kBlk - 1 + delta - kw0 < p.window);
    if (any) {
      // S = Q K^T and dP = dO V^T (lane: key, 16 rows)
      f32x16 sacc = f32x16{}, dpacc = f32x16{};
#pragma unroll
      for (int c = 0; c < T::KC; ++c) {
        sacc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(row_frag<D>(lds, qoff, lane, c), kb[c], sacc, 0, 0, 0);
        dpacc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(row_frag<D>(lds, ooff, lane, c), vb[c], dpacc, 0, 0, 0);
      }
      float pr[16], ds[16];
#pragma unroll
      for (int t = 0; t < 4; ++t) {
        // rows 4g + 8t .. +3 of the block: their lse2 and D
        const f32x4 l4 = *reinterpret_cast<const __attribute__((address_space(3))) f32x4*>(lds + loff + (4 * g + 8 * t) * 4);
        const f32x4 d4 = *reinterpret_cast<const __attribute__((address_space(3))) f32x4*>(lds + doff + (4 * g + 8 * t) * 4);
#pragma unroll
        for (int u = 0; u < 4; ++u) pr[4 * t + u] = fast_exp2(sacc[4 * t + u] * p.sl2 - l4[u]);
#pragma unroll
        for (int u = 0; u < 4; ++u) ds[4 * t + u] = dpacc[4 * t + u] - d4[u];
      }
      if (!full) {
        // register r holds row i0 + 4g + c(r), c(r) = r % 4 + 8 (r / 4); with
        // t = key - (i0 + 4g + delta): hidden by causality when t > c(r), by the
        // window when t <= c(r) - window
        const int tk = key - (i0 + 4 * g + delta);
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const int c = (r & 3) + 8 * (r >> 2);
          bool hide = p.causal && tk > c;
          if (p.window > 0 && tk <= c - p.window) hide = true;
          if (hide) pr[r] = 0.f;
        }
      }
#pragma unroll
      for (int r = 0; r < 16; ++r) ds[r] *= pr[r];
      // dV^T += dO^T P and dK^T += Q^T dS over the block's two 16-row chunks
#pragma unroll
      for (int kc = 0; kc < 2; ++kc) {
        u32x4 pp, pd;
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          pp[i] = pack_bf16x2(pr[8 * kc + 2 * i], pr[8 * kc + 2 * i + 1]);
          pd[i] = pack_bf16x2(ds[8 * kc + 2 * i], ds[8 * kc + 2 * i + 1]);
        }
        const bf16x8 bp = __builtin_bit_cast(bf16x8, pp), bd = __builtin_bit_cast(bf16x8, pd);
#pragma unroll
        for (int db = 0; db < T::NDB; ++db) {
          dvt[db] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(tr_frag<D>(lds, ooff, lane, db, kc), bp, dvt[db], 0, 0, 0);
          dkt[db] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(tr_frag<D>(lds, qoff, lane, db, kc), bd, dkt[db], 0, 0, 0);
        }
      }
    }
    // the other buffer's readers (step s - 1) passed the previous barrier
    if (s + 1 < steps) {
      stash(sets[(u + 1) % kAhead], buf ^ 1);
      fetch(sets[(u + 1) % kAhead], s + 1 + kAhead);
    }
    __syncthreads();
    return true;
   });
   if (!more) break;
  }

  // dK = scale * (dK^T)^T, dV = (dV^T)^T: lane holds key `key`, features
  // 32 db + 8 t + 4 g .. +3 in registers 4 t .. 4 t + 3.
  if (key < Nk) {
    const int64_t off = (sq.k0 + key) * kv_row + (int64_t)hk * D;
#pragma unroll
    for (int db = 0; db < T::NDB; ++db)
#pragma unroll
      for (int t = 0; t < 4; ++t) {
        const int f = 32 * db + 8 * t + 4 * g;
        u32x2 wk, wv;
        wk[0] = pack_bf16x2(dkt[db][4 * t] * p.scale, dkt[db][4 * t + 1] * p.scale);
        wk[1] = pack_bf16x2(dkt[db][4 * t + 2] * p.scale, dkt[db][4 * t + 3] * p.scale);
        wv[0] = pack_bf16x2(dvt[db][4 * t], dvt[db][4 * t + 1]);
        wv[1] = pack_bf16x2(dvt[db][4 * t + 2], dvt[db][4 * t + 3]);
        *reinterpret_cast<u32x2*>(p.dk + off + f) = wk;
        *reinterpret_cast<u32x2*>(p.dv + off + f) = wv;
      }
  }
}

// ---------------------------------------------------------------------------
// dQ.

template <int D, bool VARLEN>
__global__ __launch_bounds__(kBwdThreads) void bwd_dq_kernel(const BwdParams p) {
  using T = BT<D>;
  constexpr int KN = 64;                  // keys per step (two 32-key blocks)
  constexpr int KTILE = T::PITCH * KN;    // bytes of one staged K or V tile
  __shared__ __attribute__((aligned(16))) uint8_t smem[2 * 2 * KTILE];
  lds_u8* const lds = (lds_u8*)smem;

  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const SeqTile sq = seq_tile<VARLEN>(p, p.cu_q, p.total_q, lane);
  if (sq.tile < 0) return;  // a schedule slot past the sequence (whole group)
  const int Nq = sq.Nq, Nk = sq.Nk;
  const int qt = sq.tile, h = blockIdx.y;
  const int hk = h / p.group;
  const int q0 = qt * kBwdWaves * kBlk;
  const int qw0 = q0 + wave * kBlk;
  const int row = qw0 + (lane & 31);       // this lane's query row (column of S^T)
  const int g = lane >> 5;
  const int delta = Nk - Nq;
  const int64_t kv_row = (int64_t)p.Hkv * D;
  const int64_t q_row = (int64_t)p.Hq * D;

  bf16x8 qb[T::KC], ob[T::KC];
  float l2 = __builtin_inff(), dd = 0.f;
  {
    const int64_t off = (sq.q0 + row) * q_row + (int64_t)h * D + 8 * g;
#pragma unroll
    for (int c = 0; c < T::KC; ++c) {
      u32x4 x = {0u, 0u, 0u, 0u}, y = {0u, 0u, 0u, 0u};
      if (row < Nq) {
        x = *reinterpret_cast<const u32x4*>(p.q + off + 16 * c);
        y = *reinterpret_cast<const u32x4*>(p.dout + off + 16 * c);
      }
      qb[c] = __builtin_bit_cast(bf16x8, x);
      ob[c] = __builtin_bit_cast(bf16x8, y);
    }
    if (row < Nq) {
      const int64_t o = sq.stat(p, h, VARLEN) + row;
      l2 = p.lse2[o];
      dd = p.dsum[o];
    }
  }
  f32x16 dqt[T::NDB];
#pragma unroll
  for (int db = 0; db < T::NDB; ++db) dqt[db] = f32x16{};

  // keys some row of the tile sees: [jlo, jhi)
  const int qlast = min(Nq, q0 + kBwdWaves * kBlk) - 1;
  int jlo = 0, jhi = Nk;
  if (p.causal) jhi = min(Nk, qlast + delta + 1);
  if (p.window > 0) jlo = max(0, q0 + delta - p.window + 1);
  const int j_first = jlo & ~(KN - 1);
  const int steps = jhi > j_first ? (jhi - j_first + KN - 1) / KN : 0;

  // as in the dK/dV kernel: step t's K and V tiles travel in register set
  // t % kAhead and LDS buffer t % 2
  struct Set {
    Stage<D, KN> k, v;
  };
  Set sets[kAhead];
  const uint16_t* kbase = p.k + sq.k0 * kv_row + (int64_t)hk * D;
  const uint16_t* vbase = p.v + sq.k0 * kv_row + (int64_t)hk * D;
  const StageOff<D, KN> so(kv_row, tid);
  auto fetch = [&](Set& st, int s) __attribute__((always_inline)) {
    if (s >= steps) return;
    st.k.load(kbase, kv_row, j_first + s * KN, Nk, so);
    st.v.load(vbase, kv_row, j_first + s * KN, Nk, so);
  };
  auto stash = [&](const Set& st, int buf) __attribute__((always_inline)) {
    st.k.store(lds, (2 * buf) * KTILE, tid);
    st.v.store(lds, (2 * buf + 1) * KTILE, tid);
  };
  unroll_while<0, kAhead>([&](auto J) { fetch(sets[J], J); return true; });
  if (steps > 0) {
    stash(sets[0], 0);
    fetch(sets[0], kAhead);
  }
  __syncthreads();
  for (int s0 = 0; s0 < steps; s0 += kAhead) {
   const bool more = unroll_while<0, kAhead>([&](auto U) __attribute__((always_inline)) {
    constexpr int u = decltype(U)::value;
    const int s = s0 + u;
    if (s >= steps) return false;
    const int buf = s & 1;
    const int j0 = j_first + s * KN;
    const uint32_t koff = (2 * buf) * KTILE, voff = (2 * buf + 1) * KTILE;
#pragma unroll
    for (int kb2 = 0; kb2 < KN / kBlk; ++kb2) {
      const int jb = j0 + kb2 * kBlk;  // first key of the 32-key block
      bool any = qw0 < Nq && jb < Nk;
      if (p.causal && jb > qw0 + kBlk - 1 + delta) any = false;
      if (p.window > 0 && qw0 + delta - (jb + kBlk - 1) >= p.window) any = false;
      const bool full = (!p.causal || jb + kBlk - 1 <= qw0 + delta) &&
                        (p.window <= 0 || qw0 + kBlk - 1 + delta - jb < p.window);
      if (!any) continue;
      const uint32_t kb_off = koff + kb2 * kBlk * T::PITCH, vb_off = voff + kb2 * kBlk * T::PITCH;
      // S^T = K Q^T, dP^T = V dO^T (lane: row, 16 keys)
      f32x16 sacc = f32x16{}, dpacc = f32x16{};
#pragma unroll
      for (int c = 0; c < T::KC; ++c) {
        sacc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(row_frag<D>(lds, kb_off, lane, c), qb[c], sacc, 0, 0, 0);
        dpacc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(row_frag<D>(lds, vb_off, lane, c), ob[c], dpacc, 0, 0, 0);
      }
      float pr[16], ds[16];
#pragma unroll
      for (int r = 0; r < 16; ++r) pr[r] = fast_exp2(sacc[r] * p.sl2 - l2);
      if (!full) {
        // register r holds key jb + 4g + c(r); with t = jb + 4g - (row + delta)
        // the key is past the row's position when t + c(r) > 0 and before its
        // window when t + c(r) <= -window
        const int tk = jb + 4 * g - (row + delta);
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const int c = (r & 3) + 8 * (r >> 2);
          bool hide = p.causal && tk + c > 0;
          if (p.window > 0 && tk + c <= -p.window) hide = true;
          if (hide) pr[r] = 0.f;
        }
      }
#pragma unroll
      for (int r = 0; r < 16; ++r) ds[r] = pr[r] * (dpacc[r] - dd);
      // dQ^T += K^T dS^T over the block's two 16-key chunks
#pragma unroll
      for (int kc = 0; kc < 2; ++kc) {
        u32x4 pd;
#pragma unroll
        for (int i = 0; i < 4; ++i) pd[i] = pack_bf16x2(ds[8 * kc + 2 * i], ds[8 * kc + 2 * i + 1]);
        const bf16x8 bd = __builtin_bit_cast(bf16x8, pd);
#pragma unroll
        for (int db = 0; db < T::NDB; ++db)
          dqt[db] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(tr_frag<D>(lds, kb_off, lane, db, kc), bd, dqt[db], 0, 0, 0);
      }
    }
    // the other buffer's readers (block s - 1) passed the previous barrier
    if (s + 1 < steps) {
      stash(sets[(u + 1) % kAhead], buf ^ 1);
      fetch(sets[(u + 1) % kAhead], s + 1 + kAhead);
    }
    __syncthreads();
    return true;
   });
   if (!more) break;
  }

  if (row < Nq) {
    const int64_t off = (sq.q0 + row) * q_row + (int64_t)h * D;
#pragma unroll
    for (int db = 0; db < T::NDB; ++db)
#pragma unroll
      for (int t = 0; t < 4; ++t) {
        const int f = 32 * db + 8 * t + 4 * g;
        u32x2 w;
        w[0] = pack_bf16x2(dqt[db][4 * t] * p.scale, dqt[db][4 * t + 1] * p.scale);
        w[1] = pack_bf16x2(dqt[db][4 * t + 2] * p.scale, dqt[db][4 * t + 3] * p.scale);
        *reinterpret_cast<u32x2*>(p.dq + off + f) = w;
      }
  }
}

}  // namespace

size_t bwd_workspace_bytes(int B, int Hq, int Nq) {
  const size_t n = (size_t)B * Hq * Nq;
  return 2 * ((n * sizeof(float) + 255) / 256 * 256);
}

namespace {

// the three kernels in order; an empty grid is not launched (with no query
// rows the dK/dV kernel still writes zeros, with no keys the dQ kernel does)
template <bool VARLEN>
hipError_t launch_bwd(const BwdParams& p, int d, long long rows, dim3 g1, dim3 g2,
                      hipStream_t stream) {
  const int rpb = 256 / (d / 8);
  const long long nb = (rows + rpb - 1) / rpb;
  const dim3 g0((unsigned)(nb < 65536 ? nb : 65536));
  if (rows > 0) {
    if (d == 128)
      hipLaunchKernelGGL((bwd_prep_kernel<128, VARLEN>), g0, dim3(256), 0, stream, p);
    else
      hipLaunchKernelGGL((bwd_prep_kernel<64, VARLEN>), g0, dim3(256), 0, stream, p);
  }
  if ((long long)g1.x * g1.y * g1.z > 0) {
    if (d == 128)
      hipLaunchKernelGGL((bwd_dkdv_kernel<128, VARLEN>), g1, dim3(kBwdThreads), 0, stream, p);
    else
      hipLaunchKernelGGL((bwd_dkdv_kernel<64, VARLEN>), g1, dim3(kBwdThreads), 0, stream, p);
  }
  if ((long long)g2.x * g2.y * g2.z > 0) {
    if (d == 128)
      hipLaunchKernelGGL((bwd_dq_kernel<128, VARLEN>), g2, dim3(kBwdThreads), 0, stream, p);
    else
      hipLaunchKernelGGL((bwd_dq_kernel<64, VARLEN>), g2, dim3(kBwdThreads), 0, stream, p);
  }
  return hipGetLastError();
}

BwdParams common_params(const void* q, const void* k, const void* v, const void* out,
                        const void* dout, const float* lse, void* dq, void* dk, void* dv,
                        int Hq, int Hkv, int causal, int window, float scale, void* workspace,
                        size_t stat_rows) {
  BwdParams p{};
  p.q = static_cast<const uint16_t*>(q);
  p.k = static_cast<const uint16_t*>(k);
  p.v = static_cast<const uint16_t*>(v);
  p.o = static_cast<const uint16_t*>(out);
  p.dout = static_cast<const uint16_t*>(dout);
  p.lse = lse;
  p.dq = static_cast<uint16_t*>(dq);
  p.dk = static_cast<uint16_t*>(dk);
  p.dv = static_cast<uint16_t*>(dv);
  char* ws = static_cast<char*>(workspace);
  p.dsum = reinterpret_cast<float*>(ws);
  p.lse2 = reinterpret_cast<float*>(ws + (stat_rows * sizeof(float) + 255) / 256 * 256);
  p.Hq = Hq;
  p.Hkv = Hkv;
  p.group = Hq / Hkv;
  p.causal = causal;
  p.window = window;
  p.scale = scale;
  p.sl2 = scale * kLog2e;
  return p;
}

}  // namespace

hipError_t launch_bwd_bf16(const BwdArgs& a, hipStream_t stream) {
  BwdParams p = common_params(a.q, a.k, a.v, a.out, a.dout, a.lse, a.dq, a.dk, a.dv, a.Hq,
                              a.Hkv, a.causal, a.window, a.scale, a.workspace,
                              (size_t)a.B * a.Hq * a.Nq);
  p.B = a.B;
  p.Nq = a.Nq;
  p.Nk = a.Nk;
  constexpr int TILE = kBwdWaves * kBlk;
  const dim3 g1((a.Nk + TILE - 1) / TILE, a.Hkv, a.B);
  const dim3 g2((a.Nq + TILE - 1) / TILE, a.Hq, a.B);
  return launch_bwd<false>(p, a.d, (long long)a.B * a.Nq * a.Hq, g1, g2, stream);
}

hipError_t launch_bwd_bf16_varlen(const BwdVarlenArgs& a, hipStream_t stream) {
  BwdParams p = common_params(a.q, a.k, a.v, a.out, a.dout, a.lse, a.dq, a.dk, a.dv, a.Hq,
                              a.Hkv, a.causal, a.window, a.scale, a.workspace,
                              (size_t)a.Hq * a.total_q);
  p.cu_q = a.cu_seqlens_q;
  p.cu_k = a.cu_seqlens_k;
  p.n_seqs = a.n_seqs;
  p.total_q = a.total_q;
  p.total_k = a.total_k;
  p.B = 1;
  constexpr int TILE = kBwdWaves * kBlk;
  const dim3 g1(a.n_seqs > 0 ? a.total_k / TILE + a.n_seqs : 0, a.Hkv, 1);
  const dim3 g2(a.n_seqs > 0 ? a.total_q / TILE + a.n_seqs : 0, a.Hq, 1);
  return launch_bwd<true>(p, a.d, (long long)a.total_q * a.Hq, g1, g2, stream);
}

}  // namespace attn
