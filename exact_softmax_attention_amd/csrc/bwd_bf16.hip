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
//   bwd_dkdv   one work group per (128-key tile, KV head, batch), eight waves
//              in two roles on v_mfma_f32_32x32x16_bf16.  Producers (waves
//              0-3, 32 keys each, K and V held as A operands) form, per 32-row
//              query block of each of the G query heads,
//                S^T = K Q^T,  dP^T = V dO^T   B = Q, dO rows from LDS
//              (lane l: query row l % 32, 16 keys), then P and dS, which go
//              to LDS as bf16 [row][key] tiles.  Consumers (waves 4-7, on the
//              same SIMDs) add
//                dV^T += dO^T P   A = dO^T from the LDS transposing load
//                dK^T += Q^T dS   A = Q^T likewise, B = the tiles, read with
//              the same transposing load so that the MFMA k index runs over
//              the query rows in the same permuted order on both operands.
//   bwd_dq     one work group per 128-row query tile of one head, the same
//              two roles: producers hold Q and dO as B operands (lane l: row
//              l % 32) and form S^T = K Q^T, dP^T = V dO^T and dS^T over
//              64-key steps (A = K, V rows from LDS); consumers add
//              dQ^T += K^T dS^T (A = K^T from the transposing load).
// The consumers stage the tiles with buffer loads that write LDS directly,
// two steps ahead of their use.  The 16-byte pieces of a staged row are
// XOR-swizzled (BT::swz), which keeps both the row reads and the transposing
// reads of the same tile free of bank conflicts.
#include <type_traits>

#include "device_common.h"
#include "launch.h"

namespace attn {
namespace {

typedef short s16x4 __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) s16x4 lds_s16x4;
typedef __attribute__((address_space(3))) uint8_t lds_u8;
typedef int i32x4 __attribute__((ext_vector_type(4)));

// Buffer resource for raw 32-bit addressing: loads at byte offsets >= bytes
// return zero and touch no memory.
__device__ __forceinline__ i32x4 dma_rsrc(const void* base, uint32_t bytes) {
  const uint64_t a = reinterpret_cast<uint64_t>(base);
  i32x4 r;
  r[0] = static_cast<int>(static_cast<uint32_t>(a));
  r[1] = static_cast<int>(static_cast<uint32_t>(a >> 32) & 0xffffu);
  r[2] = static_cast<int>(bytes);
  r[3] = 0x00020000;
  return r;
}

// Loads that write LDS directly: 16 (dma16) or 4 (dma4) bytes per active
// lane from the buffer at byte offset voffset to LDS address lds + 16 x lane
// (4 x lane).  The compiler does not see them: the kernel waits for them
// itself (wait_vm) before the barrier that hands the data to other waves.
// M0 (the LDS address of the load) is set inside the asm; nothing else in
// this file uses M0.
__device__ __forceinline__ void dma16(i32x4 rsrc, int voffset, uint32_t lds) {
  asm volatile("s_mov_b32 m0, %2\n\ts_nop 0\n\tbuffer_load_dwordx4 %0, %1, 0 offen lds"
               :: "v"(voffset), "s"(rsrc), "s"(lds) : "memory", "m0");
}
__device__ __forceinline__ void dma4(i32x4 rsrc, int voffset, uint32_t lds) {
  asm volatile("s_mov_b32 m0, %2\n\ts_nop 0\n\tbuffer_load_dword %0, %1, 0 offen lds"
               :: "v"(voffset), "s"(rsrc), "s"(lds) : "memory", "m0");
}

// s_waitcnt vmcnt(N) (N < 16) with the other counters left alone.
template <int N>
__device__ __forceinline__ void wait_vm() {
  static_assert(N >= 0 && N < 16, "vmcnt field");
  __builtin_amdgcn_s_waitcnt(0x0F70 | N);
}

constexpr int kTileBlocks = 4;  // 32-row blocks per 128-row tile, one per producer wave
constexpr int kBlk = 32;  // MFMA block: 32 keys x 32 query rows

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

// The grid position (x tile or slot, y head, z sequence) a work group works
// on.  The launch's ids are remapped with xcd_remap, so that each XCD runs one
// contiguous run of (x, y, z) in order: the tiles of a head then run side by
// side on one XCD and share its L2 for the rows they all stream (Q, dO and
// the row statistics for dK/dV; K and V for dQ).  `reverse` takes a head's
// tiles last to first (dQ: under a causal mask the last query tiles see the
// most keys, and the longest work should start first).
struct Wg {
  int x, y, z;
};

__device__ __forceinline__ Wg wg_coords(bool reverse) {
  const int gx = gridDim.x, gy = gridDim.y;
  const int pid = blockIdx.x + gx * (blockIdx.y + gy * blockIdx.z);
  const int m = xcd_remap(pid, gx * gy * (int)gridDim.z);
  Wg w;
  w.x = m % gx;
  w.y = (m / gx) % gy;
  w.z = m / (gx * gy);
  if (reverse) w.x = gx - 1 - w.x;
  return w;
}

// The sequence and 128-row tile of work group `w`.  Dense: sequence w.z, tile
// w.x.  Packed: w.x is a slot of the packed axis (queries or keys, `cu` and
// `total`), the slots of sequence s starting at cu[s] / 128 + s; tile < 0 for
// a slot past the sequence's tiles.
struct SeqTile {
  int b, tile, Nq, Nk;
  int64_t q0, k0;  // first query and key row of the sequence
  __device__ int64_t stat(const BwdParams& p, int h, bool packed) const {  // LSE index of row 0
    return packed ? (int64_t)h * p.total_q + q0 : ((int64_t)b * p.Hq + h) * Nq;
  }
};

template <bool VARLEN>
__device__ __forceinline__ SeqTile seq_tile(const BwdParams& p, const Wg& w, const int* cu,
                                            int total, int lane) {
  SeqTile t;
  if constexpr (VARLEN) {
    constexpr int TILE = kTileBlocks * kBlk;
    const int slot = w.x;
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
    t.b = w.z;
    t.tile = w.x;
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
  static constexpr int PITCH = 2 * D;          // LDS bytes per staged row (no padding)
  // 16-byte piece swizzle (XOR on the piece index) of a staged row.  The LDS
  // serves 256 bytes (its 64 banks) at a time: 16 lanes of a 16-byte row read
  // or 32 lanes of an 8-byte transposing read.  Row reads take one piece of
  // 16 consecutive rows, so the swizzle must differ on each of them; the
  // transposing reads take 64 bytes (4 pieces) of 4 consecutive rows, which
  // the swizzle must move to 4 different quarters of the 256 bytes.  D = 128
  // (a row is 256 bytes): bits 2-3 follow row % 4, bits 0-1 row / 4 % 4.
  // D = 64 (two rows per 256 bytes): bit 2 follows row / 2 % 2, bits 0-1
  // row / 4 % 4.
  __device__ static int swz(int row) {
    return D == 128 ? (((row & 3) << 2) | ((row >> 2) & 3))
                    : ((((row >> 1) & 1) << 2) | ((row >> 2) & 3));
  }
  static constexpr int ROWB = 2 * D;           // global bytes per row
  static constexpr int PIECES = ROWB / 16;     // 16-byte pieces per row
};

// ---------------------------------------------------------------------------
// Shared tile helpers.

// A operand (rows x k) of a 32x32x16 MFMA from a staged tile: lane l reads row
// l % 32, features 16c + 8 (l / 32) .. +7 (piece 2c + l / 32 of the row).
template <int D>
__device__ __forceinline__ bf16x8 row_frag(const lds_u8* lds, uint32_t off, int lane, int c) {
  const int row = lane & 31;
  const uint32_t a = off + row * BT<D>::PITCH + (((2 * c + (lane >> 5)) ^ BT<D>::swz(row)) << 4);
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
  // features 32 db + 16 (G16 % 2) + 4 (s16 % 4): piece 4 db + 2 (G16 % 2) +
  // (s16 % 4) / 2, byte 8 (s16 % 2) within it; the second read is 8 rows on
  const int piece = 4 * db + 2 * (G16 & 1) + ((s16 & 3) >> 1);
  const uint32_t a = off + row * BT<D>::PITCH + ((piece ^ BT<D>::swz(row)) << 4) + 8 * (s16 & 1);
  const uint32_t b = off + (row + 8) * BT<D>::PITCH + ((piece ^ BT<D>::swz(row + 8)) << 4) + 8 * (s16 & 1);
  const s16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4*)(lds + a));
  const s16x4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4*)(lds + b));
  return __builtin_bit_cast(bf16x8, __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7));
}

// A 32 x 32 bf16 tile [row][key] with 64-byte rows, the 8-byte chunk j (keys
// 4j .. 4j + 3) of row r stored at chunk j ^ (r / 4 % 8): the XOR spreads both
// the producers' writes (row per lane, 4 keys per write) and the
// transposing reads below over all 64 banks.
__device__ __forceinline__ uint32_t ptile_chunk(int row, int chunk) {
  return (uint32_t)(row * 64 + ((chunk ^ ((row >> 2) & 7)) << 3));
}

// B operand (rows x keys) of a 32x32x16 MFMA from such a tile, row chunk kc:
// the transposing read of tr_frag, so lane l gets key l % 32 and rows
// {4g..4g+3, 8+4g..8+4g+3} + 16 kc, the row order of tr_frag's A operand.
__device__ __forceinline__ bf16x8 ptile_frag(const lds_u8* lds, uint32_t off, int lane, int kc) {
  const int G16 = lane >> 4, s16 = lane & 15;
  const int row = kc * 16 + (G16 >> 1) * 4 + (s16 >> 2);
  const int chunk = 4 * (G16 & 1) + (s16 & 3);
  const s16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4*)(lds + off + ptile_chunk(row, chunk)));
  const s16x4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4*)(lds + off + ptile_chunk(row + 8, chunk)));
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
    // O is read once (non-temporal); dO is read again by the dK/dV and dQ kernels
    const u32x4 a = *reinterpret_cast<const u32x4*>(p.dout + r * D + sub * 8);
    const u32x4 b = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(p.o + r * D + sub * 8));
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

constexpr int kDkdvWaves = 8;  // 4 producer waves + 4 consumer waves
constexpr int kDkdvThreads = kDkdvWaves * 64;

// One work group per (128-key tile, KV head, batch), 8 waves in two roles
// sharing the tile's keys (wave w and w + 4 own keys 32 (w % 4) .. +31 and
// run on one SIMD):
//   producer (waves 0-3) holds its keys' K and V rows as A operands and, for
//     query block s, forms S^T = K Q^T and dP^T = V dO^T (a lane per query
//     row, so each lane needs one row's lse2 and D), then P and dS = P (dP - D),
//     which it leaves in LDS as [row][key] bf16 tiles that the consumer reads
//     with transposing loads as the B operands of its products;
//   consumer (waves 4-7) holds the dK^T and dV^T accumulators and, for block
//     s - 1, adds dO^T P and Q^T dS (A: the transposed tiles from LDS); it also
//     stages the Q and dO tiles and the rows' lse2 and D, with loads that
//     write LDS directly, two blocks ahead.
// Each wave fits half a SIMD's registers, so the two roles' MFMAs, softmax
// and loads overlap on the SIMD.  Per iteration s: producers work on block s
// (tile buffer s % 4, probability buffer s % 2), consumers on block s - 1;
// the consumers start the loads of block s + 2 into tile buffer (s + 2) % 4
// (last read in iteration s - 1) and wait for those of block s + 1 before
// the iteration's one barrier.
template <int D, bool VARLEN>
__global__ __launch_bounds__(kDkdvThreads) void bwd_dkdv_kernel(const BwdParams p) {
  using T = BT<D>;
  constexpr int QTILE = T::PITCH * kBlk;     // bytes of one staged 32-row tile
  constexpr int kTB = 4;                     // tile buffers (Q, dO, lse2, D)
  constexpr int TBUF = 2 * QTILE + 2 * kBlk * 4;
  constexpr int PW = 2 * 32 * 64;            // one wave's P and dS tiles: 32 rows x 64 bytes each
  __shared__ __attribute__((aligned(1024))) uint8_t smem[kTB * TBUF + 2 * 4 * PW];
  lds_u8* const lds = (lds_u8*)smem;
  const uint32_t lds0 = static_cast<uint32_t>(reinterpret_cast<uintptr_t>(lds));
  constexpr uint32_t pbuf0 = kTB * TBUF;

  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const bool producer = wave < 4;
  const int kw = wave & 3;                       // key block of this wave
  const Wg wg = wg_coords(false);
  const SeqTile sq = seq_tile<VARLEN>(p, wg, p.cu_k, p.total_k, lane);
  if (sq.tile < 0) return;  // a schedule slot past the sequence (whole group)
  const int Nq = sq.Nq, Nk = sq.Nk;
  const int kt = sq.tile, hk = wg.y;
  const int k0 = kt * 4 * kBlk;                  // first key of the tile
  const int kw0 = k0 + kw * kBlk;                // first key of this wave's block
  const int key = kw0 + (lane & 31);             // this lane's key (column)
  const int g = lane >> 5;
  const int delta = Nk - Nq;
  const int64_t kv_row = (int64_t)p.Hkv * D;
  const int64_t q_row = (int64_t)p.Hq * D;

  // query rows that see some key of the tile: [qlo, qhi)
  const int klast = min(Nk, k0 + 4 * kBlk) - 1;
  int qlo = 0, qhi = Nq;
  if (p.causal) qlo = max(0, k0 - delta);
  if (p.window > 0) qhi = min(Nq, klast - delta + p.window);
  const int nblk = qhi > qlo ? (qhi - (qlo & ~(kBlk - 1)) + kBlk - 1) / kBlk : 0;
  const int q_first = qlo & ~(kBlk - 1);
  const int steps = nblk * p.group;  // (head, block) pairs, head-major

  // does this wave's 32 x 32 block of step s hold any visible pair, and does it need a mask?
  auto block_case = [&](int s, bool& any, bool& full) __attribute__((always_inline)) {
    const int i0 = q_first + (s % nblk) * kBlk;
    any = kw0 < Nk;
    if (p.causal && kw0 > i0 + kBlk - 1 + delta) any = false;
    if (p.window > 0 && i0 + delta - (kw0 + kBlk - 1) >= p.window) any = false;
    full = (!p.causal || kw0 + kBlk - 1 <= i0 + delta) &&
           (p.window <= 0 || i0 + kBlk - 1 + delta - kw0 < p.window);
  };
  // this wave's P (which = 0) or dS (1) tile of block s
  auto pt = [&](int s, int which) __attribute__((always_inline)) {
    return pbuf0 + (uint32_t)(s & 1) * 4 * PW + kw * PW + (uint32_t)which * (PW / 2);
  };

  if (producer) {
    // K and V of the lane's key as A operands (features 16c + 8g .. +7)
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
    __syncthreads();  // the consumers' first tile is in LDS
    for (int s = 0; s <= steps; ++s) {
      if (s < steps) {
        bool any, full;
        block_case(s, any, full);
        if (any) {
          const int i0 = q_first + (s % nblk) * kBlk;
          const int b = s % kTB;
          const uint32_t qoff = b * TBUF, ooff = qoff + QTILE;
          const uint32_t loff = qoff + 2 * QTILE, doff = loff + kBlk * 4;
          // S^T = K Q^T and dP^T = V dO^T: lane l holds query row i0 + n
          // (n = l % 32) and keys kw0 + 4g + c(r), c(r) = r % 4 + 8 (r / 4).  All
          // of the block's operand reads go out before the first product, so
          // that the products wait for the LDS once rather than once each.
          const int n = lane & 31;
          bf16x8 qa[T::KC], oa[T::KC];
#pragma unroll
          for (int c = 0; c < T::KC; ++c) {
            qa[c] = row_frag<D>(lds, qoff, lane, c);
            oa[c] = row_frag<D>(lds, ooff, lane, c);
          }
          const float l2 = *reinterpret_cast<const __attribute__((address_space(3))) float*>(lds + loff + n * 4);
          const float dd = *reinterpret_cast<const __attribute__((address_space(3))) float*>(lds + doff + n * 4);
          f32x16 sacc = f32x16{}, dpacc = f32x16{};
          __builtin_amdgcn_s_setprio(1);
#pragma unroll
          for (int c = 0; c < T::KC; ++c) {
            sacc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(kb[c], qa[c], sacc, 0, 0, 0);
            dpacc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(vb[c], oa[c], dpacc, 0, 0, 0);
          }
          __builtin_amdgcn_sched_group_barrier(0x100, 2 * T::KC, 0);  // the reads
          __builtin_amdgcn_sched_group_barrier(0x008, 2 * T::KC, 0);  // then the products
          __builtin_amdgcn_s_setprio(0);
          float pr[16], ds[16];
#pragma unroll
          for (int r = 0; r < 16; ++r) pr[r] = fast_exp2(sacc[r] * p.sl2 - l2);
          if (!full) {
            // with t = kw0 + 4g - (i0 + n + delta), key kw0 + 4g + c(r) is past
            // the row's position when t + c(r) > 0 and before its window when
            // t + c(r) <= -window
            const int tk = kw0 + 4 * g - (i0 + n + delta);
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
          // P and dS into this wave's [row][key] tiles: registers 4t .. 4t + 3
          // are keys 8t + 4g .. +3, chunk 2t + g of row n
#pragma unroll
          for (int t = 0; t < 4; ++t) {
            u32x2 pp, pd;
            pp[0] = pack_bf16x2(pr[4 * t], pr[4 * t + 1]);
            pp[1] = pack_bf16x2(pr[4 * t + 2], pr[4 * t + 3]);
            pd[0] = pack_bf16x2(ds[4 * t], ds[4 * t + 1]);
            pd[1] = pack_bf16x2(ds[4 * t + 2], ds[4 * t + 3]);
            const uint32_t a = ptile_chunk(n, 2 * t + g);
            *reinterpret_cast<__attribute__((address_space(3))) u32x2*>(lds + pt(s, 0) + a) = pp;
            *reinterpret_cast<__attribute__((address_space(3))) u32x2*>(lds + pt(s, 1) + a) = pd;
          }
        }
      }
      __syncthreads();
    }
    return;
  }

  // consumer: stages the tiles and accumulates dK^T, dV^T
  const int cw = kw;  // consumer wave 0..3
  f32x16 dkt[T::NDB], dvt[T::NDB];
#pragma unroll
  for (int db = 0; db < T::NDB; ++db) dkt[db] = dvt[db] = f32x16{};
  // Block t lands in tile buffer t % 4.  Each 1 KiB load of a tile fills LDS
  // bytes [1024 i, 1024 i + 1024) of it: lane L's 16 bytes go to row
  // r = (1024 i + 16 L) / PITCH, physical piece c, so the lane fetches logical
  // piece c ^ swz(r) of row r (the swizzled layout the fragment reads
  // expect).  Consumer wave cw issues loads cw * LPT .. + LPT - 1 of each
  // tile; waves 0 and 1 also load the block's lse2 and D (half a wave each).
  // Rows past Nq read as zero: zero Q and dO rows add nothing to dK and dV
  // whatever their probabilities, and lse2 = D = 0 keeps those finite.
  constexpr int NLD = QTILE / 1024;  // loads per tile
  constexpr int LPT = NLD / 4;       // per consumer wave
  static_assert(LPT * 4 == NLD, "every consumer wave moves the same share of a tile");
  int voff[LPT];
#pragma unroll
  for (int j = 0; j < LPT; ++j) {
    const int pos = (cw * LPT + j) * 1024 + lane * 16;
    const int r = pos / T::PITCH, c = (pos % T::PITCH) >> 4;
    voff[j] = r * (int)(q_row * 2) + ((c ^ T::swz(r)) << 4);
  }
  // the loads of block t into tile buffer `buf`; past the last block they
  // read zero-size ranges, so every wave issues the same loads every step
  auto issue = [&](int t, int buf) __attribute__((always_inline)) {
    const bool on = t < steps;
    const int tc = on ? t : 0;
    const int h = hk * p.group + tc / nblk;
    const int i0 = q_first + (tc % nblk) * kBlk;
    const int real = min(kBlk, Nq - i0);  // rows of the block that exist (>= 1 if on)
    const uint32_t bytes = on ? (uint32_t)((real - 1) * q_row * 2 + 2 * D) : 0u;
    const int64_t row0 = (sq.q0 + i0) * q_row + (int64_t)h * D;
    const i32x4 rq = dma_rsrc(p.q + row0, bytes), ro = dma_rsrc(p.dout + row0, bytes);
    const uint32_t lb = lds0 + (uint32_t)buf * TBUF + (uint32_t)cw * LPT * 1024;
#pragma unroll
    for (int j = 0; j < LPT; ++j) dma16(rq, voff[j], lb + j * 1024);
#pragma unroll
    for (int j = 0; j < LPT; ++j) dma16(ro, voff[j], lb + QTILE + j * 1024);
    if (cw < 2) {
      const float* st = (cw == 0 ? p.lse2 : p.dsum) + sq.stat(p, h, VARLEN) + i0;
      const i32x4 rs = dma_rsrc(st, on ? (uint32_t)real * 4 : 0u);
      const uint32_t ls = lds0 + (uint32_t)buf * TBUF + 2 * QTILE + (uint32_t)cw * kBlk * 4;
      if (lane < kBlk) dma4(rs, lane * 4, ls);
    }
  };
  // this wave's loads of the older of the two blocks in flight have landed
  auto wait_older = [&]() __attribute__((always_inline)) {
    if (cw < 2)
      wait_vm<2 * LPT + 1>();
    else
      wait_vm<2 * LPT>();
  };
  issue(0, 0);
  issue(1, 1);
  wait_older();
  __syncthreads();
  for (int s0 = 0; s0 <= steps; s0 += kTB) {
   const bool more = unroll_while<0, kTB>([&](auto U) __attribute__((always_inline)) {
    constexpr int u = decltype(U)::value;  // s % 4
    const int s = s0 + u;
    if (s > steps) return false;
    issue(s + 2, (u + 2) % kTB);
    if (s >= 1) {
      // dV^T += dO^T P and dK^T += Q^T dS of block s - 1
      bool any, full;
      block_case(s - 1, any, full);
      if (any) {
        constexpr uint32_t qoff = (uint32_t)((u + kTB - 1) % kTB) * TBUF, ooff = qoff + QTILE;
#pragma unroll
        for (int kc = 0; kc < 2; ++kc) {
          const bf16x8 bpv = ptile_frag(lds, pt(s - 1, 0), lane, kc);
          const bf16x8 bdv = ptile_frag(lds, pt(s - 1, 1), lane, kc);
          // the four dV products, then the four dK products: consecutive
          // products share their B operand (fewer switching bits)
#pragma unroll
          for (int db = 0; db < T::NDB; ++db)
            dvt[db] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(tr_frag<D>(lds, ooff, lane, db, kc), bpv, dvt[db], 0, 0, 0);
#pragma unroll
          for (int db = 0; db < T::NDB; ++db)
            dkt[db] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(tr_frag<D>(lds, qoff, lane, db, kc), bdv, dkt[db], 0, 0, 0);
        }
      }
    }
    wait_older();  // block s + 1, read by the producers after this barrier
    __syncthreads();
    return true;
   });
   if (!more) break;
  }

  // the loads past the last step (zero-size ranges) have landed before the wave ends
  __builtin_amdgcn_s_waitcnt(0x0F70);  // vmcnt(0)
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

// One work group per 128-row query tile of one head, 8 waves in the two roles
// of the dK/dV kernel (wave w and w + 4 own rows 32 (w % 4) .. +31):
//   producer (waves 0-3) holds its rows' Q and dO as B operands and, for key
//     step s (two 32-key blocks), forms S^T = K Q^T and dP^T = V dO^T, then
//     dS^T, which it leaves in LDS as bf16 B operands;
//   consumer (waves 4-7) holds the dQ^T accumulators, adds K^T dS^T of step
//     s - 1 (A: the transposed K tile from LDS) and stages the K/V tiles.
template <int D, bool VARLEN>
__global__ __launch_bounds__(kDkdvThreads) void bwd_dq_kernel(const BwdParams p) {
  using T = BT<D>;
  constexpr int KN = 64;                  // keys per step (two 32-key blocks)
  constexpr int KTILE = T::PITCH * KN;    // bytes of one staged K or V tile
  constexpr int kTB = 4;                  // tile buffers (K and V)
  constexpr int PW = 2 * 2 * 64 * 16;     // one wave's dS^T operands: [block][kc][lane] x 16 bytes
  __shared__ __attribute__((aligned(1024))) uint8_t smem[kTB * 2 * KTILE + 2 * 4 * PW];
  static_assert(sizeof(smem) <= 160 * 1024, "LDS budget");
  lds_u8* const lds = (lds_u8*)smem;
  const uint32_t lds0 = static_cast<uint32_t>(reinterpret_cast<uintptr_t>(lds));
  constexpr uint32_t pbuf0 = kTB * 2 * KTILE;

  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const bool producer = wave < 4;
  const int rw = wave & 3;                 // row block of this wave
  const Wg wg = wg_coords(true);
  const SeqTile sq = seq_tile<VARLEN>(p, wg, p.cu_q, p.total_q, lane);
  if (sq.tile < 0) return;  // a schedule slot past the sequence (whole group)
  const int Nq = sq.Nq, Nk = sq.Nk;
  const int qt = sq.tile, h = wg.y;
  const int hk = h / p.group;
  const int q0 = qt * 4 * kBlk;
  const int qw0 = q0 + rw * kBlk;
  const int row = qw0 + (lane & 31);       // this lane's query row (column of S^T)
  const int g = lane >> 5;
  const int delta = Nk - Nq;
  const int64_t kv_row = (int64_t)p.Hkv * D;
  const int64_t q_row = (int64_t)p.Hq * D;

  // keys some row of the tile sees: [jlo, jhi)
  const int qlast = min(Nq, q0 + 4 * kBlk) - 1;
  int jlo = 0, jhi = Nk;
  if (p.causal) jhi = min(Nk, qlast + delta + 1);
  if (p.window > 0) jlo = max(0, q0 + delta - p.window + 1);
  const int j_first = jlo & ~(KN - 1);
  const int steps = jhi > j_first ? (jhi - j_first + KN - 1) / KN : 0;

  // does this wave's 32 x 32 block (key block kb2 of step s) hold any visible pair / need a mask?
  auto block_case = [&](int s, int kb2, bool& any, bool& full) __attribute__((always_inline)) {
    const int jb = j_first + s * KN + kb2 * kBlk;
    any = qw0 < Nq && jb < Nk;
    if (p.causal && jb > qw0 + kBlk - 1 + delta) any = false;
    if (p.window > 0 && qw0 + delta - (jb + kBlk - 1) >= p.window) any = false;
    full = (!p.causal || jb + kBlk - 1 <= qw0 + delta) &&
           (p.window <= 0 || qw0 + kBlk - 1 + delta - jb < p.window);
  };
  auto pb = [&](int s, int kb2, int kc) __attribute__((always_inline)) {
    return pbuf0 + (uint32_t)(s & 1) * 4 * PW + rw * PW + (uint32_t)((kb2 * 2 + kc) * 64 + lane) * 16;
  };

  if (producer) {
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
    __syncthreads();  // the consumers' first tiles are in LDS
    for (int s = 0; s <= steps; ++s) {
      if (s < steps) {
        const int b = s % kTB;
        const uint32_t koff = (2 * b) * KTILE, voff = (2 * b + 1) * KTILE;
#pragma unroll
        for (int kb2 = 0; kb2 < KN / kBlk; ++kb2) {
          bool any, full;
          block_case(s, kb2, any, full);
          if (!any) continue;
          const int jb = j_first + s * KN + kb2 * kBlk;
          const uint32_t kb_off = koff + kb2 * kBlk * T::PITCH, vb_off = voff + kb2 * kBlk * T::PITCH;
          // S^T = K Q^T, dP^T = V dO^T (lane: row, 16 keys), the operand reads
          // first as in the dK/dV kernel
          bf16x8 ka[T::KC], va[T::KC];
#pragma unroll
          for (int c = 0; c < T::KC; ++c) {
            ka[c] = row_frag<D>(lds, kb_off, lane, c);
            va[c] = row_frag<D>(lds, vb_off, lane, c);
          }
          f32x16 sacc = f32x16{}, dpacc = f32x16{};
          __builtin_amdgcn_s_setprio(1);
#pragma unroll
          for (int c = 0; c < T::KC; ++c) {
            sacc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(ka[c], qb[c], sacc, 0, 0, 0);
            dpacc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(va[c], ob[c], dpacc, 0, 0, 0);
          }
          __builtin_amdgcn_sched_group_barrier(0x100, 2 * T::KC, 0);
          __builtin_amdgcn_sched_group_barrier(0x008, 2 * T::KC, 0);
          __builtin_amdgcn_s_setprio(0);
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
          // dS^T as the consumer's B operands (the block's two 16-key chunks)
#pragma unroll
          for (int kc = 0; kc < 2; ++kc) {
            u32x4 pd;
#pragma unroll
            for (int i = 0; i < 4; ++i) pd[i] = pack_bf16x2(ds[8 * kc + 2 * i], ds[8 * kc + 2 * i + 1]);
            *reinterpret_cast<__attribute__((address_space(3))) u32x4*>(lds + pb(s, kb2, kc)) = pd;
          }
        }
      }
      __syncthreads();
    }
    return;
  }

  // consumer: stages the K/V tiles and accumulates dQ^T
  const int cw = rw;  // consumer wave 0..3
  f32x16 dqt[T::NDB];
#pragma unroll
  for (int db = 0; db < T::NDB; ++db) dqt[db] = f32x16{};
  // Step t's K and V tiles land in tile buffer t % 4 through loads that write
  // LDS directly, each lane fetching the swizzled piece that belongs at its
  // LDS position (as in the dK/dV kernel); consumer wave cw issues loads
  // cw * LPT .. + LPT - 1 of each tile.  Keys past Nk read as zero, and zero
  // K and V rows add nothing to dQ.
  constexpr int NLD = KTILE / 1024;  // loads per tile
  constexpr int LPT = NLD / 4;       // per consumer wave
  static_assert(LPT * 4 == NLD, "every consumer wave moves the same share of a tile");
  int voff[LPT];
#pragma unroll
  for (int j = 0; j < LPT; ++j) {
    const int pos = (cw * LPT + j) * 1024 + lane * 16;
    const int r = pos / T::PITCH, c = (pos % T::PITCH) >> 4;
    voff[j] = r * (int)(kv_row * 2) + ((c ^ T::swz(r)) << 4);
  }
  const uint16_t* kbase = p.k + sq.k0 * kv_row + (int64_t)hk * D;
  const uint16_t* vbase = p.v + sq.k0 * kv_row + (int64_t)hk * D;
  // the loads of step t into tile buffer `buf`; past the last step they read
  // zero-size ranges, so every wave issues the same loads every step
  auto issue = [&](int t, int buf) __attribute__((always_inline)) {
    const bool on = t < steps;
    const int j0 = j_first + (on ? t : 0) * KN;
    const int real = min(KN, Nk - j0);  // keys of the step that exist (>= 1 if on)
    const uint32_t bytes = on ? (uint32_t)((real - 1) * kv_row * 2 + 2 * D) : 0u;
    const i32x4 rk = dma_rsrc(kbase + (int64_t)j0 * kv_row, bytes);
    const i32x4 rv = dma_rsrc(vbase + (int64_t)j0 * kv_row, bytes);
    const uint32_t lb = lds0 + (uint32_t)buf * 2 * KTILE + (uint32_t)cw * LPT * 1024;
#pragma unroll
    for (int j = 0; j < LPT; ++j) dma16(rk, voff[j], lb + j * 1024);
#pragma unroll
    for (int j = 0; j < LPT; ++j) dma16(rv, voff[j], lb + KTILE + j * 1024);
  };
  issue(0, 0);
  issue(1, 1);
  wait_vm<2 * LPT>();  // step 0's tiles (step 1's may be in flight)
  __syncthreads();
  for (int s0 = 0; s0 <= steps; s0 += kTB) {
   const bool more = unroll_while<0, kTB>([&](auto U) __attribute__((always_inline)) {
    constexpr int u = decltype(U)::value;  // s % 4
    const int s = s0 + u;
    if (s > steps) return false;
    // step s + 2 into tile buffer (s + 2) % 4, last read in iteration s - 1
    issue(s + 2, (u + 2) % kTB);
    if (s >= 1) {
      constexpr int bp = (u + kTB - 1) % kTB;  // tile buffer of step s - 1
      constexpr uint32_t koff = (2 * bp) * KTILE;
#pragma unroll
      for (int kb2 = 0; kb2 < KN / kBlk; ++kb2) {
        bool any, full;
        block_case(s - 1, kb2, any, full);
        if (!any) continue;
        const uint32_t kb_off = koff + kb2 * kBlk * T::PITCH;
        // dQ^T += K^T dS^T over the block's two 16-key chunks
#pragma unroll
        for (int kc = 0; kc < 2; ++kc) {
          const bf16x8 bd = *reinterpret_cast<const __attribute__((address_space(3))) bf16x8*>(lds + pb(s - 1, kb2, kc));
#pragma unroll
          for (int db = 0; db < T::NDB; ++db)
            dqt[db] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(tr_frag<D>(lds, kb_off, lane, db, kc), bd, dqt[db], 0, 0, 0);
        }
      }
    }
    wait_vm<2 * LPT>();  // step s + 1's tiles, read by the producers after this barrier
    __syncthreads();
    return true;
   });
   if (!more) break;
  }

  __builtin_amdgcn_s_waitcnt(0x0F70);  // vmcnt(0): the loads past the last step have landed
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
  // the work-group remap indexes the grid with 32-bit ints
  constexpr long long kMaxGroups = 0x7fffffffLL;
  if ((long long)g1.x * g1.y * g1.z > kMaxGroups || (long long)g2.x * g2.y * g2.z > kMaxGroups)
    return hipErrorInvalidConfiguration;
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
      hipLaunchKernelGGL((bwd_dkdv_kernel<128, VARLEN>), g1, dim3(kDkdvThreads), 0, stream, p);
    else
      hipLaunchKernelGGL((bwd_dkdv_kernel<64, VARLEN>), g1, dim3(kDkdvThreads), 0, stream, p);
  }
  if ((long long)g2.x * g2.y * g2.z > 0) {
    if (d == 128)
      hipLaunchKernelGGL((bwd_dq_kernel<128, VARLEN>), g2, dim3(kDkdvThreads), 0, stream, p);
    else
      hipLaunchKernelGGL((bwd_dq_kernel<64, VARLEN>), g2, dim3(kDkdvThreads), 0, stream, p);
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
  constexpr int TILE = kTileBlocks * kBlk;
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
  constexpr int TILE = kTileBlocks * kBlk;
  const dim3 g1(a.n_seqs > 0 ? a.total_k / TILE + a.n_seqs : 0, a.Hkv, 1);
  const dim3 g2(a.n_seqs > 0 ? a.total_q / TILE + a.n_seqs : 0, a.Hq, 1);
  return launch_bwd<true>(p, a.d, (long long)a.total_q * a.Hq, g1, g2, stream);
}

}  // namespace attn
