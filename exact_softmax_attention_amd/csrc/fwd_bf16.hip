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
//   * 8 waves x 32 query rows = 256 rows per work group, one work group per
//     CU, so each SIMD runs two waves.  Each wave computes S^T = K Q^T with
//     v_mfma_f32_32x32x16_bf16 (A = K rows from LDS, B = its Q rows held in
//     registers for the whole loop).  In the 32x32 accumulator layout lane l
//     holds column l % 32, i.e. one query row, and 16 keys, so the row max /
//     row sum are in-lane plus one exchange with lane l ^ 32.
//   * O^T = V^T P^T, again 32x32x16: B = P^T straight from the score
//     registers (converted to bf16, round-to-nearest-even; the row sum is
//     taken over the float32 values, so LSE is exact to fp32), A = V^T read
//     with the LDS transpose load (ds_read_b64_tr_b16) from a row-major V
//     tile.  The MFMA k index is a permutation of the tile's keys, the same
//     for both operands.
//   * The two waves of a SIMD are kept in opposite phases ("ping-pong"): while
//     one issues the matrix products, the other computes its softmax on the
//     vector ALUs; a workgroup barrier swaps the phases (see the schedule
//     comment at the kernel).
//   * K/V tiles are staged global -> registers -> LDS (two slots per kind),
//     group A moving K and group B moving V during their vector phases, with
//     two tiles in flight in registers so a load has two phases to land; LDS
//     rows are padded so that the fragment reads are bank-conflict free, and
//     fragment reads run several MFMAs ahead of their use.
//   * The softmax runs stage by stage over the whole tile (32 independent
//     FMAs, then 32 exponentials, ...) with tree reductions, and the row max
//     and sum are exchanged with lane l ^ 32 by v_permlane32_swap on the
//     vector ALU rather than through LDS, which the other wave keeps busy.
//   * Tiles wholly outside the causal/window band are never visited; only
//     tiles that cut the band boundary or the key tail pay for the per-element
//     mask.  The row maximum is raised lazily (only when a row's max grows by
//     more than 2^8), so most tiles skip the accumulator rescale.
//   * Work groups are ordered heavy-first (last query tiles first) inside a
//     head and remapped so that the tiles of one head share an XCD (and its
//     L2), since they all stream the same K/V.
#include "device_common.h"
#include "launch.h"

namespace attn {
namespace {

constexpr int kWaves = 8;                    // two groups of 4, one wave of each per SIMD
constexpr int kRowsPerWave = 32;
constexpr int kBM = kWaves * kRowsPerWave;   // query rows per work group
constexpr int kThreads = kWaves * 64;
constexpr int kGroupThreads = kThreads / 2;
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
  static constexpr int CHUNKS = BN * D / 8 / kGroupThreads;  // 16-byte pieces per group thread
  static_assert(CHUNKS * kGroupThreads * 8 == BN * D, "staging must cover the tile");
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

// Schedule ("ping-pong").  The 8 waves form two groups, A = waves 0-3 and
// B = waves 4-7, so each SIMD runs one wave of each.  Every wave alternates
// an MFMA phase, M(k) = scores of tile k and P V of tile k-1, with a vector
// phase, V(k) = softmax of tile k.  Group B runs one barrier behind group A,
// so while one group keeps the matrix cores busy the other does its softmax;
// the phases swap at every barrier.  Barrier slots: A does M(k) in slot 2k
// and V(k) in 2k+1; B does M(k) in 2k+1 and V(k) in 2k+2.
//
// Staging (two K and two V slots in LDS): A, in V(k), stores K(k+1) and
// starts loading K(k+3); B, in V(k), stores V(k+1) and starts loading V(k+3)
// (register sets alternate between even and odd tiles).
// K(k+1) lands in the slot of K(k-1), last read in slot 2k-1, and is first
// read in slot 2k+2; V(k+1) lands in the slot of V(k-1), last read in slot
// 2k+1, and is first read in slot 2k+4.
//
// POS_SCALE: scale > 0, so the row maximum of scale*s is scale * max(s) and the
// scaling folds into the exponent's FMA.  Otherwise every score is scaled first.
template <int D, bool POS_SCALE>
__global__ __launch_bounds__(kThreads, 1) void fwd_bf16_kernel(const Params p) {
  using T = Tile<D>;
  __shared__ __attribute__((aligned(16))) uint16_t smem[2 * (T::K_ELEMS + T::V_ELEMS)];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const bool group_b = wave >= kWaves / 2;
  const int gtid = tid & (kGroupThreads - 1);
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
  const int n_tiles = kv_end > kv_begin ? (kv_end + T::BN - 1) / T::BN - t_begin : 0;

  // this wave's Q rows as the B operand of K Q^T (8 bf16 per k-chunk)
  const int64_t q_row = (int64_t)p.Hq * D;
  bf16x8 qf[T::KC];
  {
    const int row = min(qw0 + n, p.Nq - 1);  // rows past the end compute garbage, never stored
    const uint16_t* qp = p.q + ((int64_t)b * p.Nq + row) * q_row + (int64_t)h * D + g * 8;
#pragma unroll
    for (int c = 0; c < T::KC; ++c) qf[c] = *reinterpret_cast<const bf16x8*>(qp + c * 16);
  }

  // Staging: group A moves K tiles, group B V tiles.  Piece c of a group
  // thread is row (gtid + c*256) / (D/8) of the tile, 16-byte column
  // gtid % (D/8).  Rows past the last key re-read the last key: their scores
  // are masked and their probabilities are exactly zero, so a finite duplicate
  // contributes nothing.
  const int64_t kv_row = (int64_t)p.Hkv * D;
  const uint16_t* src = (group_b ? p.v : p.k) + (int64_t)b * p.Nk * kv_row + (int64_t)hk * D;
  const int col8 = gtid % (D / 8);
  const int row0 = gtid / (D / 8);
  constexpr int kRowStep = kGroupThreads / (D / 8);
  const int dst_stride = group_b ? T::VSTRIDE : T::KSTRIDE;
  u32x4 sreg0[T::CHUNKS], sreg1[T::CHUNKS];  // tiles of even / odd index, two in flight
  auto kslot = [&](int i) { return smem + (i & 1) * T::K_ELEMS; };
  auto vslot = [&](int i) { return smem + 2 * T::K_ELEMS + (i & 1) * T::V_ELEMS; };
  auto stage_load = [&](int k, u32x4 (&sreg)[T::CHUNKS]) {  // tile index k relative to t_begin
    const int j0 = (t_begin + k) * T::BN;
#pragma unroll
    for (int c = 0; c < T::CHUNKS; ++c) {
      const int j = min(j0 + row0 + c * kRowStep, p.Nk - 1);
      sreg[c] = *reinterpret_cast<const u32x4*>(src + (int64_t)j * kv_row + col8 * 8);
    }
  };
  auto stage_store = [&](int k, const u32x4 (&sreg)[T::CHUNKS]) {
    uint16_t* dst = group_b ? vslot(k) : kslot(k);
#pragma unroll
    for (int c = 0; c < T::CHUNKS; ++c)
      *reinterpret_cast<u32x4*>(dst + (row0 + c * kRowStep) * dst_stride + col8 * 8) = sreg[c];
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

  auto wave_skips = [&](int k) {
    const int j0 = (t_begin + k) * T::BN;
    bool skip = qw0 >= p.Nq;
    if (p.causal && j0 > qw0 + kRowsPerWave - 1 + delta) skip = true;
    if (p.window > 0 && j0 + T::BN - 1 < qw0 + delta - p.window + 1) skip = true;
    return skip;
  };

  float m_run = kNegInf;  // running row max (base-2 domain), same in lanes n and n+32
  float l_run = 0.f;      // running row sum over this lane's keys
  f32x16 acc[T::NDB];
#pragma unroll
  for (int db = 0; db < T::NDB; ++db) acc[db] = f32x16{};
  f32x16 st[T::NKB];          // scores of the tile between its M and V phases
  uint32_t pk[T::NKB][8];     // bf16 probabilities between a V phase and the next M phase

  // M(k): scores of tile k, then P V of tile k-1.  The fragment reads run a
  // few MFMAs ahead of their use so that the LDS latency stays hidden.
  auto m_phase = [&](int k) {
    __builtin_amdgcn_s_setprio(1);
    if (k < n_tiles && !wave_skips(k)) {
      const uint16_t* ks = kslot(k) + n * T::KSTRIDE + g * 8;
      constexpr int NQK = T::NKB * T::KC;  // MFMAs of the score tile
      constexpr int LA = 8;                // reads in flight ahead
      bf16x8 kf[NQK];
#pragma unroll
      for (int i = 0; i < LA; ++i)
        kf[i] = *reinterpret_cast<const bf16x8*>(ks + (i / T::KC) * 32 * T::KSTRIDE + (i % T::KC) * 16);
#pragma unroll
      for (int kb = 0; kb < T::NKB; ++kb) st[kb] = f32x16{};
#pragma unroll
      for (int i = 0; i < NQK; ++i) {
        if (i + LA < NQK)
          kf[i + LA] = *reinterpret_cast<const bf16x8*>(
              ks + ((i + LA) / T::KC) * 32 * T::KSTRIDE + ((i + LA) % T::KC) * 16);
        st[i / T::KC] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(kf[i], qf[i % T::KC], st[i / T::KC], 0, 0, 0);
      }
      // keep LA reads in flight: reads, then alternate one MFMA / one read
      __builtin_amdgcn_sched_group_barrier(0x100, LA, 0);
#pragma unroll
      for (int i = 0; i < NQK; ++i) {
        __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
        if (i + LA < NQK) __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
      }
    }
    if (k >= 1 && !wave_skips(k - 1)) {
      const uint16_t* vrow = vslot(k - 1) + vt_key * T::VSTRIDE + vt_col;
      constexpr int NPV = T::VC * T::NDB;  // MFMAs of the P V update
      constexpr int LA = 6;
      bf16x8 vf[NPV];
      auto vread = [&](int i) {  // i = kc * NDB + db
        const uint16_t* r = vrow + (i / T::NDB) * 16 * T::VSTRIDE + (i % T::NDB) * 32;
        const s16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4*)r);
        const s16x4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4*)(r + 8 * T::VSTRIDE));
        return __builtin_bit_cast(bf16x8, __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7));
      };
#pragma unroll
      for (int i = 0; i < LA; ++i) vf[i] = vread(i);
#pragma unroll
      for (int i = 0; i < NPV; ++i) {
        if (i + LA < NPV) vf[i + LA] = vread(i + LA);
        const int kc = i / T::NDB, db = i % T::NDB;
        const int kb = kc >> 1, half = kc & 1;
        u32x4 pw;
        pw[0] = pk[kb][half * 4 + 0];
        pw[1] = pk[kb][half * 4 + 1];
        pw[2] = pk[kb][half * 4 + 2];
        pw[3] = pk[kb][half * 4 + 3];
        acc[db] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(vf[i], __builtin_bit_cast(bf16x8, pw),
                                                         acc[db], 0, 0, 0);
      }
      __builtin_amdgcn_sched_group_barrier(0x100, 2 * LA, 1);
#pragma unroll
      for (int i = 0; i < NPV; ++i) {
        __builtin_amdgcn_sched_group_barrier(0x008, 1, 1);
        if (i + LA < NPV) __builtin_amdgcn_sched_group_barrier(0x100, 2, 1);
      }
    }
    __builtin_amdgcn_s_setprio(0);
  };

  // V(k): softmax of tile k (mask, lazy max, exponentials), then staging
  auto v_phase = [&](int k, u32x4 (&snext)[T::CHUNKS]) {  // snext: registers of tile k+1 (and k+3)
    if (k < n_tiles && !wave_skips(k)) {
      const int j0 = (t_begin + k) * T::BN;
      if (!POS_SCALE) {
#pragma unroll
        for (int kb = 0; kb < T::NKB; ++kb)
#pragma unroll
          for (int r = 0; r < 16; ++r) st[kb][r] *= p.sl2;
      }
      const bool need_mask = (j0 + T::BN > p.Nk) ||
                             (p.causal && j0 + T::BN - 1 > qw0 + delta) ||
                             (p.window > 0 && qw0 + kRowsPerWave - 1 + delta - j0 >= p.window);
      if (need_mask) {
        // visible keys of this lane's row, as offsets from the lane's first key
        // (key = j0 + 4g + c with c a compile-time constant per register)
        const int pos = qw0 + n + delta;
        const int base = j0 + 4 * g;
        int hi = p.Nk - 1 - base;
        if (p.causal) hi = min(hi, pos - base);
        if (p.window > 0) {
          const int lo = pos - p.window + 1 - base;
#pragma unroll
          for (int kb = 0; kb < T::NKB; ++kb)
#pragma unroll
            for (int r = 0; r < 16; ++r) {
              const int c = kb * 32 + (r >> 2) * 8 + (r & 3);
              if (c > hi || c < lo) st[kb][r] = kNegInf;
            }
        } else {
#pragma unroll
          for (int kb = 0; kb < T::NKB; ++kb)
#pragma unroll
            for (int r = 0; r < 16; ++r) {
              const int c = kb * 32 + (r >> 2) * 8 + (r & 3);
              if (c > hi) st[kb][r] = kNegInf;
            }
        }
      }
      // online softmax with a lazily raised maximum: the stored max only moves
      // when some row's max exceeds it by more than 2^8, so most tiles skip
      // the accumulator rescale; probabilities stay <= 2^8, and the final
      // division uses the sum taken at the same max, so the result is exact.
      // row max as a tree (independent chains keep the VALU pipeline full)
      float mq[4];
#pragma unroll
      for (int j = 0; j < 4; ++j) mq[j] = fmaxf(st[0][4 * j], st[0][4 * j + 1]);
#pragma unroll
      for (int kb = 0; kb < T::NKB; ++kb)
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          if (kb == 0 && (r & 3) < 2) continue;
          mq[r >> 2] = fmaxf(mq[r >> 2], st[kb][r]);
        }
      float mx = fmaxf(fmaxf(mq[0], mq[1]), fmaxf(mq[2], mq[3]));
      {  // max with lane l ^ 32 (the same row) on the VALU
        float a = mx, b = mx;
        // inline asm: the compiler folds a max of the builtin's two results away
        asm volatile("s_nop 1\n\tv_permlane32_swap_b32 %0, %1" : "+v"(a), "+v"(b));
        mx = fmaxf(a, b);
      }
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
      // exponentials in place, stage by stage, so that each stage is 32
      // independent instructions
#pragma unroll
      for (int kb = 0; kb < T::NKB; ++kb)
#pragma unroll
        for (int r = 0; r < 16; ++r)
          st[kb][r] = POS_SCALE ? fmaf(st[kb][r], p.sl2, -m_use) : st[kb][r] - m_use;
#pragma unroll
      for (int kb = 0; kb < T::NKB; ++kb)
#pragma unroll
        for (int r = 0; r < 16; ++r) st[kb][r] = fast_exp2(st[kb][r]);
#pragma unroll
      for (int kb = 0; kb < T::NKB; ++kb)
#pragma unroll
        for (int i = 0; i < 8; ++i) pk[kb][i] = pack_bf16x2(st[kb][2 * i], st[kb][2 * i + 1]);
      // float32 row sum (the LSE must reproduce exp(S - LSE) to fp32), as a tree
      float rq[4] = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int kb = 0; kb < T::NKB; ++kb)
#pragma unroll
        for (int r = 0; r < 16; ++r) rq[r & 3] += st[kb][r];
      l_run += (rq[0] + rq[1]) + (rq[2] + rq[3]);
    }
    if (k + 1 < n_tiles) stage_store(k + 1, snext);
    if (k + 3 < n_tiles) stage_load(k + 3, snext);
  };

  // prologue: K(0) in LDS; A holds K(1), B holds V(0) in registers
  if (n_tiles > 0) {
    if (!group_b) {
      stage_load(0, sreg0);
      stage_store(0, sreg0);
      if (n_tiles > 1) stage_load(1, sreg1);
      if (n_tiles > 2) stage_load(2, sreg0);
    } else {
      stage_load(0, sreg0);
    }
  }
  __syncthreads();
  if (group_b) {  // B's V(-1): store V(0), start V(1)
    if (n_tiles > 0) stage_store(0, sreg0);
    if (n_tiles > 1) stage_load(1, sreg1);
    if (n_tiles > 2) stage_load(2, sreg0);
    __syncthreads();
  }
  // Make the Q loads complete here, once: otherwise the wait for them is placed
  // inside the loop, where it also waits for the staging loads in flight.
#pragma unroll
  for (int c = 0; c < T::KC; ++c) asm volatile("" ::"v"(qf[c]));
  // two tiles per trip so that the staging registers alternate statically
  for (int k = 0; k <= n_tiles; k += 2) {
    m_phase(k);
    __syncthreads();
    v_phase(k, sreg1);
    __syncthreads();
    if (k + 1 > n_tiles) break;
    m_phase(k + 1);
    __syncthreads();
    v_phase(k + 1, sreg0);
    __syncthreads();
  }
  if (!group_b) __syncthreads();  // A's extra barrier matches B's first one

  // epilogue: O = acc / l (bf16, RNE); LSE = (m + log2 l) ln 2
  float la = l_run, lb = l_run;
  asm volatile("s_nop 1\n\tv_permlane32_swap_b32 %0, %1" : "+v"(la), "+v"(lb));
  const float l_tot = la + lb;
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
