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
//   * K/V tiles go from HBM/L2 straight into LDS with buffer loads that
//     write LDS (no registers, no LDS store instructions), into a ring of
//     kSlots tile slots per kind, so that a load has 2*(kSlots-1) phases to
//     land.  Each load instruction fills 1 KiB of LDS contiguously; the 16-byte
//     pieces of a row are XOR-swizzled (each lane fetches the piece that
//     belongs at its LDS position) so that the fragment reads of K and the
//     transposed reads of V are bank-conflict free.  Rows past the last key
//     read as zero (buffer range check).
//   * The softmax runs stage by stage over the whole tile (32 independent
//     FMAs, then 32 exponentials, ...) with tree reductions, and the row max
//     and sum are exchanged with lane l ^ 32 by v_permlane32_swap on the
//     vector ALU rather than through LDS, which the other wave keeps busy.
//   * Tiles wholly outside the causal/window band are never visited; only
//     tiles that cut the band boundary or the key tail pay for the per-element
//     mask.  The exponentials are taken against the stored row maximum, which
//     is raised only when a tile's terms would grow past 2^8, so most tiles
//     skip both the row maximum and the accumulator rescale.
//   * Work groups are ordered heavy-first (last query tiles first) inside a
//     head and remapped so that the tiles of one head share an XCD (and its
//     L2), since they all stream the same K/V.
//   * Three modes share the loop: dense [B, N, H, D] tensors; packed
//     sequences of different lengths (cu_seqlens offsets; packed sequence
//     boundaries are what "How to Reduce Attention Computation Cost in LLM
//     Training" says need variable-length kernels); and new tokens over a
//     block-paged KV cache ("Inference Engineering", 2.5), where each wave
//     loads its 8 rows of a key tile from the cache block that holds them.
#include <atomic>
#include <climits>
#include <mutex>
#include <type_traits>

#include "device_common.h"
#include "launch.h"

namespace attn {
namespace {

constexpr int kWaves = 8;                    // two groups of 4, one wave of each per SIMD
constexpr int kRowsPerWave = 32;
constexpr int kBM = kWaves * kRowsPerWave;   // query rows per work group
constexpr int kThreads = kWaves * 64;
constexpr int kSlots = 4;                    // LDS tile slots per kind (K, V)
constexpr int kSeqLds = 2048;                // packed modes: sequence-table entries kept in LDS
constexpr float kRaise = 256.0f;  // raise the stored max when a partial row sum exceeds this

typedef short s16x4 __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) s16x4 lds_s16x4;
typedef int i32x4 __attribute__((ext_vector_type(4)));

template <int D>
struct Tile {
  static constexpr int BN = 64;                      // keys per tile
  static constexpr int NKB = BN / 32;                // 32-key blocks of S^T
  static constexpr int NDB = D / 32;                 // 32-feature blocks of O^T
  static constexpr int KC = D / 16;                  // k-chunks of K Q^T
  static constexpr int VC = BN / 16;                 // k-chunks of V^T P^T
  static constexpr int ROWB = D * 2;                 // bytes of one key row in LDS
  static constexpr int TILEB = BN * ROWB;            // bytes of one K or V tile
  static constexpr int NLD = TILEB / 1024;           // 1 KiB load instructions per tile
  static constexpr int LPW = NLD / kWaves;           // per wave, per kind
  static constexpr int LDS_BYTES = 2 * kSlots * TILEB;
  static_assert(LPW * kWaves == NLD, "every wave moves the same share of a tile");
  static_assert(LDS_BYTES <= 160 * 1024, "LDS budget");
  // 16-byte piece swizzles (XOR on the piece index within a row).
  // K is read 16 bytes per lane down 16 consecutive rows at one logical
  // piece: the XOR spreads those rows over all 64 banks.  V is read with the
  // transposing load, 8 bytes per lane, 4 consecutive rows x 64 bytes per 32
  // lanes: the XOR moves each of the 4 rows to a different 64-byte quarter.
  __device__ static int kswz(int row) { return D == 128 ? (row & 15) : ((row >> 1) & 7); }
  __device__ static int vswz(int row) { return D == 128 ? ((row & 3) << 2) : (((row >> 1) & 1) << 2); }
};

struct Params {
  const uint16_t* q;
  const uint16_t* k;
  const uint16_t* v;
  uint16_t* o;
  float* lse;
  int Hq, Hkv, group, Nq, Nk, causal, window, n_qtiles, total;
  int slot;      // this launch's slot of scheduling counters
  unsigned tag;  // and its tag (see claim_unit)
  int pairing;  // work units are pairs of query tiles (see the schedule)
  // dense: query heads of one KV head that a work item holds (1: one head;
  // 2, 4 or 8, dividing the group: kBM / gpack positions of each, one head
  // per group of kWaves / gpack waves)
  int gpack;
  float sl2;  // scale * log2(e): scores are kept in the base-2 domain
  // packed sequences: boundaries of the query and key rows of each sequence,
  // the total rows of each tensor, and the schedule's tile slots per head
  const int* cu_q;
  const int* cu_k;
  int n_seqs, total_q, total_k, vtiles;
  // paged cache: k and v are [num_blocks, 16, Hkv, D]; key t of sequence s is
  // slot t % 16 of block table[s * max_blocks + t / 16]; seq_lens[s] keys
  const int* table;
  const int* seq_lens;
  int max_blocks, num_blocks;
  // paged: an item whose key tiles span several chunks of chunk_tiles tiles
  // is done as one work unit per chunk, each writing its normalised partial
  // O (fp32) and LSE to part_o [Hq][vtiles][chunks][kBM][D] and part_lse
  // [Hq][vtiles][chunks][kBM]; a merge kernel combines them
  int chunks, chunk_tiles;
  float* part_o;
  float* part_lse;
};

// What the kernel reads: dense [B, N, H, D] tensors, packed sequences
// (cu_seqlens), or packed query chunks over a paged KV cache.
enum Mode { kDense = 0, kVarlen = 1, kPaged = 2 };
constexpr int kBlockTokens = 16;  // tokens per cache block
constexpr int kChunkTiles = 128;  // paged: 64-key tiles per key chunk (8192 keys)

// Key tiles (64 keys) that query rows [i0, i0 + rows) of a sequence with Nq
// queries and Nk keys may see: [t_begin, t_begin + n_tiles).  i0 may be
// negative (packed sequences' tiles end at the sequence's last row).
struct TileRange {
  int t_begin, n_tiles;
};
__device__ __forceinline__ TileRange tile_range(int i0, int Nq, int Nk, int causal, int window,
                                                int rows = kBM) {
  const int delta = Nk - Nq;
  int kv_end = Nk;
  if (causal) kv_end = min(Nk, i0 + rows + delta);
  int kv_begin = 0;
  if (window > 0) kv_begin = max(0, max(i0, 0) + delta - window + 1);  // rows below 0 do not exist
  TileRange r;
  r.t_begin = kv_begin / 64;
  r.n_tiles = kv_end > kv_begin ? (kv_end + 63) / 64 - r.t_begin : 0;
  return r;
}

// Scheduling counters of the persistent kernel: slot s holds one unit counter
// per XCD, a 64-bit word made of the launch's tag (high half) and the next
// unit index (low half).  Every launch takes a fresh tag and a slot, and is
// preceded on its stream by a one-wave kernel that sets the slot's counters
// to (tag, 0); a work group claims units with one atomic add.  The host makes
// slot use exclusive: a launch on a slot whose previous launch may still run
// waits for it (an event recorded after each launch), and a launch captured
// into a graph gets a slot of its own (see launch()), whose set-up kernel is
// replayed with it.  Should two launches still meet on one counter (replays
// of two graphs whose captures are kGraphSlots captures apart, running at
// the same time), the tag shows it: the group then takes the counter over
// for its own launch at one past its previous claim (claims only increase,
// and under one tag the indices handed out stay a prefix [0, max], so the
// launch skips no unit; the other may, since the add already took an index).
constexpr int kXcds = 8;  // XCDs of the device; work group w runs on XCD w % 8
constexpr int kEagerSlots = 256;  // slots of launches made outside graph capture
constexpr int kGraphSlots = 4096;  // slots of captured launches, taken in turn
__device__ unsigned long long g_sched[(kEagerSlots + kGraphSlots) * kXcds];

// Next unit index of this launch from counter `w`; `last` is this group's
// previous claim (-1 before the first).
__device__ __forceinline__ int claim_unit(unsigned long long* w, unsigned tag, int last) {
  const unsigned long long old = atomicAdd(w, 1ull);
  if ((unsigned)(old >> 32) == tag && (int)(unsigned)old > last) return (int)(unsigned)old;
  // another launch's tag (or an index at or below ours after a take-over)
  unsigned long long v = __hip_atomic_load(w, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  const unsigned next = (unsigned)(last + 1);
  for (;;) {
    const unsigned have = (unsigned)v;
    const unsigned c = (unsigned)(v >> 32) == tag && have > next ? have : next;
    const unsigned long long nv = ((unsigned long long)tag << 32) | (c + 1u);
    const unsigned long long prev = atomicCAS(w, v, nv);
    if (prev == v) return (int)c;
    v = prev;
  }
}

// Sets the counters of `slot` to (tag, 0) before the launch that uses them.
__global__ __launch_bounds__(64) void sched_reset_kernel(int slot, unsigned tag) {
  if (threadIdx.x < kXcds)
    __hip_atomic_store(&g_sched[slot * kXcds + threadIdx.x], (unsigned long long)tag << 32,
                       __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

// Buffer resource for raw (unswizzled) 32-bit addressing: loads at byte
// offsets >= bytes return zero and touch no memory.
__device__ __forceinline__ i32x4 make_rsrc(const void* base, uint32_t bytes) {
  const uint64_t a = reinterpret_cast<uint64_t>(base);
  i32x4 r;
  r[0] = static_cast<int>(static_cast<uint32_t>(a));
  r[1] = static_cast<int>(static_cast<uint32_t>(a >> 32) & 0xffffu);
  r[2] = static_cast<int>(bytes);
  r[3] = 0x00020000;
  return r;
}

// 16 bytes per lane from the buffer into LDS at lds_base + OFF + 16 * lane.
// The compiler does not see this load: the kernel waits for it itself
// (wait_vm) before the barrier that hands the tile to the other waves.  M0
// (the LDS address of the load) is set inside the asm; nothing else in these
// kernels uses M0.  The scalar add also writes SCC, so SCC is declared
// clobbered: the compiler may otherwise keep a compare result in SCC across
// the asm.
template <uint32_t OFF>
__device__ __forceinline__ void load_lds16(i32x4 rsrc, int voffset, uint32_t lds_base) {
  asm volatile("s_add_u32 m0, %2, %3\n\ts_nop 0\n\tbuffer_load_dwordx4 %0, %1, 0 offen lds"
               :: "v"(voffset), "s"(rsrc), "s"(lds_base), "n"(OFF) : "memory", "m0", "scc");
}

// s_waitcnt vmcnt(N) (N < 16) with the other counters left alone.
template <int N>
__device__ __forceinline__ void wait_vm() {
  static_assert(N >= 0 && N < 16, "vmcnt field");
  __builtin_amdgcn_s_waitcnt(0x0F70 | N);
}

// Work-group barrier that orders LDS only (global memory needs no fence
// here: the LDS-writing loads are waited for explicitly).
__device__ __forceinline__ void lds_barrier() {
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "workgroup", "local");
  __builtin_amdgcn_s_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "workgroup", "local");
}

// Barrier that leaves this wave's LDS reads in flight: for reads of a slot
// that no wave rewrites before this wave has consumed them.  The empty asm
// statements keep the compiler from moving LDS accesses across it.
__device__ __forceinline__ void lds_barrier_reads_in_flight() {
  asm volatile("" ::: "memory");
  __builtin_amdgcn_s_barrier();
  asm volatile("" ::: "memory");
}

__device__ __forceinline__ int floordiv(int a, int b) {  // b > 0
  const int q = a / b;
  return (a % b != 0 && a < 0) ? q - 1 : q;
}


template <int I, int N, typename F>
__device__ __forceinline__ bool unrolled_while(F&& f) {
  if constexpr (I < N) {
    if (!f(std::integral_constant<int, I>{})) return false;
    return unrolled_while<I + 1, N>(f);
  }
  return true;
}

// Schedule ("ping-pong").  The 8 waves form two groups, A = waves 0-3 and
// B = waves 4-7, so each SIMD runs one wave of each.  Every wave alternates
// an MFMA phase, M(k) = scores of tile k and P V of tile k-1, with a vector
// phase, V(k) = softmax of tile k.  Group B runs one barrier behind group A,
// so while one group keeps the matrix cores busy the other does its softmax;
// the phases swap at every barrier.  Barrier slots: A does M(k) in slot 2k
// and V(k) in 2k+1; B does M(k) in 2k+1 and V(k) in 2k+2.
//
// Loads: "batch m" = K(m-1+S) and V(m-2+S) (S = kSlots), into the slots of
// K(m-1) and V(m-2), which were last read in slot 2m-1.  Each wave issues its
// share of batch m at the start of its own M(m): group A in slot 2m, group B
// in slot 2m+1 (the MFMA phase leaves the wave's issue slots idle).  Batch m
// is first read in slot 2m+2S-3, where group A's V(m+S-2) reads ahead the
// first operands of its M(m+S-1), so every wave waits for its own loads of
// batch m at the end of slot 2m+2S-4, before the barrier: group A at the end
// of an M phase (S-2 later batches may stay in flight), group B at the end
// of a V phase (S-3 later batches).  Loads of tiles past the last one read
// nothing and fill free slots.
//
// Softmax: the exponentials are first taken against the stored row maximum.
// The online softmax is exact for any reference value that keeps the terms
// finite, so the stored maximum only has to be raised when a term would grow
// large: when a lane's partial row sum of the tile exceeds 2^8 (or is not
// finite, as on a row's first visible tile), the tile is redone with the true
// row maximum, and the accumulator and sum are rescaled.  Most tiles skip
// the row maximum altogether.  The decision is the row's own (the wave takes
// the slow path when any row needs it, but only those rows raise), so a row's
// results do not depend on which rows share its wave or its query tile.
//
// POS_SCALE: scale > 0, so the row maximum of scale*s is scale * max(s) and the
// scaling folds into the exponent's FMA.  Otherwise every score is scaled first,
// before the mask sets hidden scores to -inf.
template <int D, bool POS_SCALE, int MODE>
__global__ __launch_bounds__(kThreads, 1) void fwd_bf16_kernel(const Params p) {
  constexpr bool VARLEN = MODE != kDense;  // queries packed by cu_seqlens
  constexpr bool PAGED = MODE == kPaged;
  using T = Tile<D>;
  constexpr int S = kSlots;
  __shared__ __attribute__((aligned(1024))) uint8_t smem[T::LDS_BYTES];
  // K slots at [0, S*TILEB), V slots at [S*TILEB, 2*S*TILEB)
  typedef __attribute__((address_space(3))) uint8_t lds_u8;
  lds_u8* const lds = (lds_u8*)smem;
  const uint32_t lds0 = static_cast<uint32_t>(reinterpret_cast<uintptr_t>(lds));

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const bool group_b = wave >= kWaves / 2;
  const int n = lane & 31;  // query row within the wave / MFMA column
  const int g = lane >> 5;  // k-half of the MFMA operands

  // Persistent schedule: one work group per CU takes work units from a queue
  // until it is empty.  With pairing, a unit is two query tiles of one head,
  // the j-th heaviest and the j-th lightest (under a causal mask all such
  // pairs cost the same), processed heavy first; otherwise a unit is one
  // query tile.  Units are ordered by head, the costliest first within a head,
  // and split over the XCDs in proportion to the work groups each XCD runs
  // (work group w runs on XCD w % 8); each XCD hands out its range through its
  // own counter.  So the groups of an XCD work on the same few heads at a time
  // (their K/V stream through the XCD's L2), and the cheap units, taken last,
  // even out the finishing times whatever the cost of each unit.  Packed
  // sequences and the paged cache (modes 1 and 2) have no pairing: a unit is
  // one query tile of one head of one sequence (paged: and one key chunk),
  // found from the unit index as described at the item setup below.
  constexpr int kXcd = kXcds;
  __shared__ int s_unit;  // the next unit, broadcast from thread 0
  __shared__ int s_bad;   // paged: some wave met a block it cannot read
  // Packed modes: the sequence table (cu_seqlens_q, and cu_seqlens_k or the
  // paged lengths) is copied into LDS once per work group when it fits, so
  // that an item finds its sequence and sizes without global loads.
  typedef const __attribute__((address_space(3))) int lds_cint;
  __shared__ int s_seq_a[VARLEN ? kSeqLds : 1], s_seq_b[VARLEN ? kSeqLds : 1];
  const bool seq_in_lds = VARLEN && p.n_seqs + 1 <= kSeqLds;
  if (seq_in_lds) {
    for (int i = tid; i <= p.n_seqs; i += kThreads) {
      s_seq_a[i] = p.cu_q[i];
      s_seq_b[i] = PAGED ? (i < p.n_seqs ? p.seq_lens[i] : 0) : p.cu_k[i];
    }
  }
  const int G = gridDim.x;
  const int xcd = blockIdx.x % kXcd;
  int groups_before = 0;
  for (int x = 0; x < xcd; ++x) groups_before += (G - x + kXcd - 1) / kXcd;
  const int Gx = (G - xcd + kXcd - 1) / kXcd;
  const int nq = p.n_qtiles;
  const int per_head = p.pairing ? (nq + 1) / 2 : nq;
  const int gp = (MODE == kDense && p.gpack > 1) ? p.gpack : 1;  // query heads per item
  const int units = VARLEN ? p.total : p.total / nq * per_head;
  const int first = (int)((int64_t)units * groups_before / G);
  const int last = (int)((int64_t)units * (groups_before + Gx) / G);
  unsigned long long* const ctr = g_sched + p.slot * kXcd + xcd;
  int claimed = -1;  // thread 0: this group's latest claim
  if (tid == 0) {
    claimed = claim_unit(ctr, p.tag, claimed);
    s_unit = first + claimed;
  }
  __syncthreads();
  for (int unit = s_unit; unit < last;) {
  int grabbed = 0;  // the unit after this one, in flight meanwhile
  if (tid == 0) {
    claimed = claim_unit(ctr, p.tag, claimed);
    grabbed = claimed;
  }
  const int bh = unit / per_head;
  // pairs: the middle (costliest under a window) first; tiles: heavy first
  const int j = per_head - 1 - (unit - bh * per_head);
  for (int e = 0; e < 2; ++e) {
    if (e == 1 && (VARLEN || !p.pairing || j == nq - 1 - j)) break;
    if (PAGED && tid == 0) s_bad = 0;  // read by the previous item before the unit's last barrier
    // this item: query tile qt of head h of sequence b, whose Nq query rows
    // start at token row q_tok0 and Nk key rows at k_tok0
    int b, h, qt, Nq, Nk, i0;
    int64_t q_tok0, k_tok0, lse0;
    bool bad = false;  // paged: a length or block id the kernel cannot read
    int slot = 0, chunk = 0;  // packed: schedule slot; paged: key chunk
    if constexpr (VARLEN) {
      // unit = (KV head, tile slot, query head within the group); the slots
      // of sequence s start at cu_q[s] / kBM + s, which leaves room for its
      // tiles (heaviest first), and a slot past them is skipped
      const int hg = unit % p.group;
      int rest = unit / p.group;
      if constexpr (PAGED) {  // the chunks of one item are neighbours in the queue
        chunk = rest % p.chunks;
        rest /= p.chunks;
      }
      slot = rest % p.vtiles;
      h = (rest / p.vtiles) * p.group + hg;
      // (the copy above precedes the first __syncthreads)
      int cq0, cq1;
      if (seq_in_lds) {
        b = find_seq<kBM>((lds_cint*)s_seq_a, p.n_seqs, p.total_q, slot, lane);
        cq0 = __builtin_amdgcn_readfirstlane(s_seq_a[b]);  // uniform: scalar registers
        cq1 = __builtin_amdgcn_readfirstlane(s_seq_a[b + 1]);
      } else {
        b = find_seq<kBM>(p.cu_q, p.n_seqs, p.total_q, slot, lane);
        cq0 = p.cu_q[b];
        cq1 = p.cu_q[b + 1];
      }
      const int q0 = clampi(cq0, 0, p.total_q);
      const int q1 = clampi(cq1, q0, p.total_q);
      Nq = q1 - q0;
      int k0 = 0;
      if constexpr (PAGED) {
        // the chunk's queries are the last Nq of the sequence's seq_len tokens
        const int len = seq_in_lds ? __builtin_amdgcn_readfirstlane(s_seq_b[b]) : p.seq_lens[b];
        bad = len < 0 || len > p.max_blocks * kBlockTokens;
        Nk = bad ? 0 : len;
        // A block id outside the pool anywhere in the sequence's table makes
        // the whole sequence NaN, as a bad length does: every item of the
        // sequence finds it here, whichever blocks the item itself reads (the
        // tile and chunk split is kept, so the merge pass sees NaN partials).
        // The ids are checked again where blocks are read.
        if (!bad) {
          const int nblk = (len + kBlockTokens - 1) / kBlockTokens;
          const int* const ids = p.table + (int64_t)b * p.max_blocks;
          bool out = false;
          for (int i = lane; i < nblk; i += 64) out |= (unsigned)ids[i] >= (unsigned)p.num_blocks;
          bad = __builtin_amdgcn_ballot_w64(out) != 0;
        }
      } else {
        const int ck0 = seq_in_lds ? __builtin_amdgcn_readfirstlane(s_seq_b[b]) : p.cu_k[b];
        const int ck1 = seq_in_lds ? __builtin_amdgcn_readfirstlane(s_seq_b[b + 1]) : p.cu_k[b + 1];
        k0 = clampi(ck0, 0, p.total_k);
        Nk = clampi(ck1, k0, p.total_k) - k0;
      }
      const int off = slot - (q0 / kBM + b);
      const int ntl = (Nq + kBM - 1) / kBM;
      if (off < 0 || off >= ntl) {
        // every wave has read s_unit before thread 0 writes the next unit
        // (a real item passes several barriers in between)
        __syncthreads();
        break;
      }
      qt = ntl - 1 - off;
      // Packed sequences: the tiles end at the sequence's last row (tile off
      // holds rows [Nq - (off + 1) kBM, Nq - off kBM)), so the partial tile
      // holds the first rows, which see the fewest keys under a causal mask;
      // its rows below 0 do not exist (never stored).  The paged mode keeps
      // tiles from row 0 (its chunk merge addresses rows by tile).
      i0 = PAGED ? qt * kBM : Nq - (off + 1) * kBM;
      q_tok0 = q0;
      k_tok0 = k0;
      lse0 = (int64_t)h * p.total_q + q0;
    } else {
      // Grouped heads (gp > 1): the item holds positions [i0, i0 + kBM / gp)
      // of gp query heads that share a KV head (gp divides the group),
      // kWaves / gp waves per head, so its key range is that of kBM / gp
      // positions (less of the causal diagonal and of a window's edge
      // computed for nothing)
      qt = p.pairing ? (e == 0 ? nq - 1 - j : j) : nq - 1 - (per_head - 1 - j);
      i0 = qt * (kBM / gp);
      const int nhb = p.Hq / gp;  // head blocks
      b = bh / nhb;
      h = (bh - b * nhb) * gp + wave / (kWaves / gp);  // this wave's query head
      Nq = p.Nq;
      Nk = p.Nk;
      q_tok0 = (int64_t)b * Nq;
      k_tok0 = (int64_t)b * Nk;
      lse0 = ((int64_t)b * p.Hq + h) * Nq;
    }
    const int hk = h / p.group;
    const int qw0 = i0 + (wave % (kWaves / gp)) * kRowsPerWave;  // this wave's first row
    const int delta = Nk - Nq;

    static_assert(T::BN == 64, "tile_range counts 64-key tiles");
    const TileRange tr_ = tile_range(i0, Nq, Nk, p.causal, p.window, kBM / gp);
    int t_begin = tr_.t_begin;
    int n_tiles = tr_.n_tiles;
    bool split = false;  // paged: this unit does one chunk of the item's tiles
    if constexpr (PAGED) {
      const int c0 = n_tiles > 0 ? t_begin / p.chunk_tiles : 0;
      const int c1 = n_tiles > 0 ? (t_begin + n_tiles - 1) / p.chunk_tiles : 0;
      if (chunk < c0 || chunk > c1) {
        __syncthreads();  // as for a skipped slot: s_unit is read before it is rewritten
        break;
      }
      split = c1 > c0;
      if (split) {
        const int lo = max(t_begin, chunk * p.chunk_tiles);
        const int hi = min(t_begin + n_tiles, (chunk + 1) * p.chunk_tiles);
        t_begin = lo;
        n_tiles = hi - lo;
      }
    }

    // this wave's Q rows as the B operand of K Q^T (8 bf16 per k-chunk)
    const int64_t q_row = (int64_t)p.Hq * D;
    bf16x8 qf[T::KC];
    {
      const int row = max(0, min(qw0 + n, Nq - 1));  // rows outside [0, Nq) compute garbage, never stored
      const uint16_t* qp = p.q + (q_tok0 + row) * q_row + (int64_t)h * D + g * 8;
  #pragma unroll
      for (int c = 0; c < T::KC; ++c) qf[c] = *reinterpret_cast<const bf16x8*>(qp + c * 16);
    }

    // ---- loads into LDS.  Instruction i of a tile fills LDS bytes
    // [1024 i, 1024 i + 1024) of the slot; lane L's 16 bytes land at 1024 i + 16 L,
    // which is row r = (1024 i + 16 L) / ROWB, physical piece c; the lane
    // fetches logical piece c ^ swizzle(r) of key row r.
    const int64_t kv_row = (int64_t)p.Hkv * D;                 // elements between keys
    const uint32_t kv_row_b = static_cast<uint32_t>(kv_row * 2);
    const int64_t head_off = PAGED ? (int64_t)hk * D : k_tok0 * kv_row + (int64_t)hk * D;
    const uint16_t* kbase = p.k + head_off;
    const uint16_t* vbase = p.v + head_off;
    int koff[T::LPW], voff[T::LPW];
  #pragma unroll
    for (int j = 0; j < T::LPW; ++j) {
      const int pos = (wave * T::LPW + j) * 1024 + lane * 16;
      const int r = pos / T::ROWB;
      const int c = (pos % T::ROWB) >> 4;
      // paged: the wave's rows (8 consecutive) lie in one cache block
      const int rr = PAGED ? (r & (kBlockTokens - 1)) : r;
      koff[j] = rr * (int)kv_row_b + ((c ^ T::kswz(r)) << 4);
      voff[j] = rr * (int)kv_row_b + ((c ^ T::vswz(r)) << 4);
    }
    // Each wave issues the tiles of one kind in order (K(0), K(1), ... and
    // V(0), V(1), ...), so a running byte address per kind is enough; the range
    // of a tile is whole except for the last visible one, and zero past it.
    const uint32_t lds_wave = lds0 + wave * T::LPW * 1024;
    const uint32_t tile_b = (uint32_t)T::BN * kv_row_b;  // bytes of a whole tile's rows
    uint32_t last_b = 0;  // bytes of the last visible tile: up to the end of key row Nk-1
    if (n_tiles > 0) {
      const int rows = Nk - (t_begin + n_tiles - 1) * T::BN;  // >= 1
      last_b = rows >= T::BN ? tile_b : (uint32_t)(rows - 1) * kv_row_b + T::ROWB;
    }
    const uint8_t* knext = reinterpret_cast<const uint8_t*>(kbase) + (int64_t)t_begin * tile_b;
    const uint8_t* vnext = reinterpret_cast<const uint8_t*>(vbase) + (int64_t)t_begin * tile_b;
    int kt = 0, vt = 0;  // index of the next tile of each kind
    // Paged cache: this wave's 8 rows of a 64-key tile lie in logical block
    // 4 t' + wave / 2 (t' = t_begin + t), rows 8 (wave % 2) .. +7 of it.  A
    // block is looked up only when some of its keys exist (so the table is
    // never read past the sequence); a needed id outside the pool marks the
    // item bad and is not read.
    static_assert(T::LPW * 1024 / T::ROWB == 8, "8 rows per wave and tile");
    constexpr int kNone = INT_MIN;
    // read through the constant address space: the index is uniform, so these
    // become scalar loads (lgkmcnt), which do not wait behind the vector
    // memory counter that paces the tile loads
    typedef const __attribute__((address_space(4))) int const_int;
    const_int* const trow = (const_int*)(PAGED ? p.table + (int64_t)b * p.max_blocks : p.table);
    const int64_t blk_b = (int64_t)kBlockTokens * kv_row * 2;  // bytes per cache block
    auto lookup = [&](int t) __attribute__((always_inline)) {
      const int lb = (t_begin + t) * (T::BN / kBlockTokens) + (wave >> 1);
      return (t < n_tiles && lb * kBlockTokens < Nk) ? trow[lb] : kNone;
    };
    auto paged_rsrc = [&](const uint16_t* base, int id, int t) __attribute__((always_inline)) {
      const int lb = (t_begin + t) * (T::BN / kBlockTokens) + (wave >> 1);
      const int nv = min(Nk - lb * kBlockTokens, kBlockTokens);  // keys in the block (> 0 if looked up)
      const bool ok = id != kNone && (unsigned)id < (unsigned)p.num_blocks;
      bad |= id != kNone && !ok;
      const uint32_t bytes = ok ? (uint32_t)(nv - 1) * kv_row_b + T::ROWB : 0u;
      return make_rsrc(reinterpret_cast<const uint8_t*>(base) + (ok ? (int64_t)id * blk_b : 0), bytes);
    };
    auto issue = [&](auto DST, const uint8_t*& next, int& t, const int (&off)[T::LPW]) {
      constexpr uint32_t dst = decltype(DST)::value;
      const uint32_t bytes = t < n_tiles - 1 ? tile_b : (t == n_tiles - 1 ? last_b : 0u);
      i32x4 rsrc;
      if constexpr (PAGED) {
        const bool is_k = dst < S * T::TILEB;
        rsrc = paged_rsrc(is_k ? kbase : vbase, lookup(t), t);
      } else {
        rsrc = make_rsrc(next, bytes);
      }
      load_lds16<dst>(rsrc, off[0], lds_wave);
      if constexpr (T::LPW > 1) load_lds16<dst + 1024>(rsrc, off[1], lds_wave);
      static_assert(T::LPW <= 2, "load count per wave");
      next += tile_b;
      ++t;
    };
    auto rsrc_of = [&](const uint8_t* next, int t) __attribute__((always_inline)) {
      const uint32_t bytes = t < n_tiles - 1 ? tile_b : (t == n_tiles - 1 ? last_b : 0u);
      return make_rsrc(next, bytes);
    };
    // the next K tile into K slot SLOT, the next V tile into V slot SLOT
    auto issue_k = [&](auto SLOT) __attribute__((always_inline)) {
      issue(std::integral_constant<uint32_t, decltype(SLOT)::value * T::TILEB>{}, knext, kt, koff);
    };
    auto issue_v = [&](auto SLOT) __attribute__((always_inline)) {
      issue(std::integral_constant<uint32_t, (S + decltype(SLOT)::value) * T::TILEB>{}, vnext, vt, voff);
    };
    using std::integral_constant;
    // paged: buffer resources of the next M phase's K and V loads (K tile kt,
    // V tile kt - 1), made at the start of each V phase from block ids looked
    // up one phase earlier, so the scalar loads of the table never stall the
    // matrix phase
    i32x4 prk = {}, prv = {};
    int id_k = kNone, id_next = kNone;  // ids of K tile kt - 1 and of tile kt
    auto paged_advance = [&]() __attribute__((always_inline)) {
      prv = paged_rsrc(vbase, id_k, kt - 1);
      id_k = id_next;
      prk = paged_rsrc(kbase, id_k, kt);
      id_next = lookup(kt + 1);
    };

    // ---- LDS fragment offsets (bytes from the LDS base, per lane; slots and
    // blocks are added as immediates)
    // K: row n of the 32-key block, logical piece 2 kc + g, which sits at
    // piece (2kc + g) ^ swz(n) = (g ^ swz(n)) ^ 2kc: the fragment of k-chunk kc
    // is at kfrag0 ^ (kc << 5) (the row term has no bits there)
    const uint32_t kfrag0 = n * T::ROWB + ((g ^ T::kswz(n)) << 4);
    // V (transposing read): for MFMA k-chunk kc and feature block db, lane
    // (group G = lane/16, s = lane%16) points at key kc*16 + (G/2)*4 + s/4
    // (+8 for the second read) and features db*32 + 16*(G%2) + 4*(s%4).  The
    // hardware hands lane 4r+c of each 16-lane group the 4 keys of source lanes
    // r, r+4, r+8, r+12 at feature 4r+c, which is V^T in the operand layout, with
    // lane group g holding keys {g*4..g*4+3, 8+g*4..8+g*4+3} of the chunk.
    // The swizzle of a key row depends only on the key modulo 4.
    const int G16 = lane >> 4, s16 = lane & 15;
    const int vt_key = (G16 >> 1) * 4 + (s16 >> 2);
    uint32_t vaddr[T::NDB];
  #pragma unroll
    for (int db = 0; db < T::NDB; ++db) {
      const int piece = db * 4 + 2 * (G16 & 1) + ((s16 & 3) >> 1);
      vaddr[db] = S * T::TILEB + vt_key * T::ROWB + ((piece ^ T::vswz(vt_key)) << 4) + 8 * (s16 & 1);
    }

    // Tiles [kf0, kf1) are visible to every row of this wave and need no mask.
    int kf0 = 0, kf1 = 0;
    if (qw0 < Nq) {
      int hi = min(n_tiles, Nk / T::BN - t_begin);  // before the key tail
      if (p.causal) hi = min(hi, floordiv(qw0 + delta + 1, T::BN) - t_begin);
      int lo = 0;
      if (p.window > 0) lo = max(0, -floordiv(p.window - qw0 - kRowsPerWave - delta, T::BN) - t_begin);
      kf0 = lo;
      kf1 = max(lo, hi);
    }
    auto wave_skips = [&](int k) __attribute__((always_inline)) {
      const int j0 = (t_begin + k) * T::BN;
      bool skip = qw0 >= Nq || qw0 + kRowsPerWave - 1 < 0;
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
    u32x4 pk[T::VC];            // bf16 probabilities between a V phase and the next M
                                // phase, as the B operands of the V^T P^T k-chunks
  #pragma unroll
    for (int kc = 0; kc < T::VC; ++kc) pk[kc] = u32x4{};

    constexpr int NQK = T::NKB * T::KC;  // MFMAs of the score tile
    constexpr int NPV = T::VC * T::NDB;  // MFMAs of the P V update
    constexpr int LA = 8;                // MFMAs whose operands are read ahead
    static_assert(LA <= NQK, "the read-ahead starts with score operands");
    // Score MFMA i takes k-chunk kc = i / NKB of key block kb = i % NKB: the
    // key blocks of one k-chunk are issued back to back, so consecutive MFMAs
    // share their Q operand (fewer operand bits switch: the kernel is power
    // limited).  K fragment i of the tile in K slot `slot`:
    auto kfrag = [&](int slot, int i) __attribute__((always_inline)) {
      const int kc = i / T::NKB, kb = i % T::NKB;
      const uint32_t a = (kfrag0 ^ (kc << 5)) + slot * T::TILEB + kb * 32 * T::ROWB;
      return *reinterpret_cast<const __attribute__((address_space(3))) bf16x8*>(lds + a);
    };
    // score operands read ahead across the barrier, at the end of the V
    // phase (deeper read-ahead measured no faster and costs 4 registers per
    // fragment)
    constexpr int NPRE = NQK < 8 ? NQK : 8;
    bf16x8 kpre[NPRE];

    // M(k): scores of tile k, then P V of tile k-1, as one stream of MFMAs
    // whose LDS fragment reads run LA MFMAs ahead (the V reads start while the
    // score MFMAs still run).  U = k mod S (compile time), so every LDS slot
    // offset is an immediate.  M(0) (FIRST) has no P V half.
    auto m_phase = [&](auto U, auto FIRST, int k, int& vcase) __attribute__((always_inline)) {
      constexpr int u = decltype(U)::value;
      constexpr int NM = decltype(FIRST)::value ? NQK : NQK + NPV;  // MFMAs of this phase
      // case of tile k for the V phase (scalar work, done here where the
      // issue slots are idle): 0 no mask, 1 masked, 2 not visible
      constexpr int ks = u;                // slot of K(k)
      constexpr int vs = (u + S - 1) % S;  // slot of V(k-1)
      constexpr uint32_t kdst = ((u + S - 1) % S) * T::TILEB;        // batch k
      constexpr uint32_t vdst = (S + (u + S - 2) % S) * T::TILEB;
      i32x4 rk, rv;
      // The loads of batch k and the scalar work, one piece after each of the
      // first MFMAs: issued in one block they held up the matrix pipe, since
      // a wave issues in order.
      static_assert(T::LPW == 1 || T::LPW == 2, "load count per wave");
      auto piece = [&](int j) __attribute__((always_inline)) {
        if (j == 0) {
          if constexpr (PAGED) rk = prk; else rk = rsrc_of(knext, kt);
          load_lds16<kdst>(rk, koff[0], lds_wave);
        }
        if (j == 1) {
          if constexpr (T::LPW > 1) load_lds16<kdst + 1024>(rk, koff[1], lds_wave);
          knext += tile_b;
          ++kt;
        }
        if (j == 2) {
          if constexpr (PAGED) rv = prv; else rv = rsrc_of(vnext, vt);
          load_lds16<vdst>(rv, voff[0], lds_wave);
        }
        if (j == 3) {
          if constexpr (T::LPW > 1) load_lds16<vdst + 1024>(rv, voff[1], lds_wave);
          vnext += tile_b;
          ++vt;
        }
        if (j == 4) {
          vcase = (unsigned)(k - kf0) < (unsigned)(kf1 - kf0) ? 0 : (k < n_tiles && !wave_skips(k)) ? 1 : 2;
          asm volatile("" : "+s"(vcase));
        }
      };
      bf16x8 kf[NQK], vf[NPV];
      auto kread = [&](int i) __attribute__((always_inline)) { kf[i] = kfrag(ks, i); };
      auto vread = [&](int i) __attribute__((always_inline)) {  // i = kc * NDB + db
        const uint32_t a = vaddr[i % T::NDB] + vs * T::TILEB + (i / T::NDB) * 16 * T::ROWB;
        const s16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4*)(lds + a));
        const s16x4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4*)(lds + a + 8 * T::ROWB));
        vf[i] = __builtin_bit_cast(bf16x8, __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7));
      };
      auto qk_mfma = [&](int i) __attribute__((always_inline)) {  // the first k-chunk starts from zero
        const int kc = i / T::NKB, kb = i % T::NKB;
        st[kb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(kf[i], qf[kc], kc == 0 ? f32x16{} : st[kb],
                                                         0, 0, 0);
      };
      auto pv_mfma = [&](int i) __attribute__((always_inline)) {
        const int kc = i / T::NDB, db = i % T::NDB;
        acc[db] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(vf[i], __builtin_bit_cast(bf16x8, pk[kc]),
                                                         acc[db], 0, 0, 0);
      };
      // Both halves always run: a tile this wave does not see has all-zero
      // probabilities (set by its V phase), and the scores of a tile it will
      // not use are simply not read.  Skipping saves no time, since every wave
      // waits at the same barriers.
      // MFMA j < NQK is score MFMA j, else P V MFMA j - NQK; its operands are
      // read before MFMA j - LA, except the first NPRE, which were read at the
      // end of this wave's previous V phase (kpre): the matrix pipe starts at
      // once and the score MFMAs do not wait on LDS.
      auto read = [&](int j) __attribute__((always_inline)) { if (j < NQK) kread(j); else vread(j - NQK); };
  #pragma unroll
      for (int j = 0; j < NPRE; ++j) kf[j] = kpre[j];
      static_assert(NQK >= 5, "the loads ride on the score MFMAs");
  #pragma unroll
      for (int j = 0; j < NM; ++j) {
        if (j + LA < NM && j + LA >= NPRE) read(j + LA);
        if (j < NQK) qk_mfma(j); else pv_mfma(j - NQK);
        if (j < 5) piece(j);
      }
  #pragma unroll
      for (int j = 0; j < NM; ++j) {
        __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
        if (j + LA < NQK && j + LA >= NPRE)
          __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
        else if (j + LA >= NQK && j + LA < NM)
          __builtin_amdgcn_sched_group_barrier(0x100, 2, 0);
      }
      if (!group_b) wait_vm<2 * T::LPW * (S - 2)>();
    };

    // Masking in place: key offset c (a compile-time constant per register, key
    // = j0 + 4g + c) is hidden when c > hi (causal diagonal, key tail) or c < lo
    // (window).  The compare/select pair is written in asm with the score tied
    // to its own register, so that masked and unmasked tiles leave the scores
    // where the MFMAs wrote them (the compiler otherwise copies them to merge
    // the two paths).
    auto mask_above = [&](int hi) __attribute__((always_inline)) {
  #pragma unroll
      for (int kb = 0; kb < T::NKB; ++kb)
  #pragma unroll
        for (int r = 0; r < 16; ++r) {
          const int c = kb * 32 + (r >> 2) * 8 + (r & 3);
          asm("v_cmp_gt_i32 vcc, %1, %2\n\tv_cndmask_b32 %0, %0, %3, vcc"
              : "+v"(st[kb][r]) : "n"(c), "v"(hi), "v"(kNegInf) : "vcc");
        }
    };
    auto mask_below = [&](int lo) __attribute__((always_inline)) {
  #pragma unroll
      for (int kb = 0; kb < T::NKB; ++kb)
  #pragma unroll
        for (int r = 0; r < 16; ++r) {
          const int c = kb * 32 + (r >> 2) * 8 + (r & 3);
          asm("v_cmp_lt_i32 vcc, %1, %2\n\tv_cndmask_b32 %0, %0, %3, vcc"
              : "+v"(st[kb][r]) : "n"(c), "v"(lo), "v"(kNegInf) : "vcc");
        }
    };

    // exponentials of the tile against the reference max mref (base-2
    // domain), packed to bf16 pairs; returns this lane's float32 partial row sum
    auto exp_tile = [&](float mref) __attribute__((always_inline)) {
      float e[T::NKB][16];
  #pragma unroll
      for (int kb = 0; kb < T::NKB; ++kb)
  #pragma unroll
        for (int r = 0; r < 16; ++r) e[kb][r] = fast_exp2(fmaf(st[kb][r], POS_SCALE ? p.sl2 : 1.f, -mref));
  #pragma unroll
      for (int kb = 0; kb < T::NKB; ++kb)
  #pragma unroll
        for (int i = 0; i < 8; ++i) pk[kb * 2 + (i >> 2)][i & 3] = pack_bf16x2(e[kb][2 * i], e[kb][2 * i + 1]);
      float rq[4] = {e[0][0], e[0][1], e[0][2], e[0][3]};
  #pragma unroll
      for (int kb = 0; kb < T::NKB; ++kb)
  #pragma unroll
        for (int r = (kb == 0 ? 4 : 0); r < 16; ++r) rq[r & 3] += e[kb][r];
      return (rq[0] + rq[1]) + (rq[2] + rq[3]);
    };

    // V(k): softmax of tile k (mask, exponentials, occasional max update)
    auto v_phase = [&](auto U, int k, int vcase) __attribute__((always_inline)) {
      (void)U;
      if constexpr (PAGED) paged_advance();
      if (vcase != 2) {
        if constexpr (!POS_SCALE) {
          // scale <= 0: the scores are scaled before the mask (a masked score
          // must be -inf after scaling, and -inf times a scale <= 0 is not)
  #pragma unroll
          for (int kb = 0; kb < T::NKB; ++kb)
  #pragma unroll
            for (int r = 0; r < 16; ++r) st[kb][r] *= p.sl2;
        }
        if (vcase == 1) {
          const int j0 = (t_begin + k) * T::BN;
          const int pos = qw0 + n + delta;  // this lane's row position
          const int base = j0 + 4 * g;      // key of offset 0 in this lane
          if ((j0 + T::BN > Nk) || (p.causal && j0 + T::BN - 1 > qw0 + delta)) {
            int hi = Nk - 1 - base;
            if (p.causal) hi = min(hi, pos - base);
            mask_above(hi);
          }
          if (p.window > 0 && qw0 + kRowsPerWave - 1 + delta - j0 >= p.window)
            mask_below(pos - p.window + 1 - base);
        }
        // fast path: against the stored max (m_run = -inf gives inf/NaN sums)
        float ls = exp_tile(m_run);
        const bool need = !(ls <= kRaise);
        if (__builtin_amdgcn_ballot_w64(need) != 0) {
          // row max of the scaled scores as a tree
          auto sv = [&](int kb, int r) __attribute__((always_inline)) {
            return st[kb][r];  // (scale <= 0: already scaled)
          };
          float mq[4];
  #pragma unroll
          for (int j = 0; j < 4; ++j) mq[j] = fmaxf(sv(0, 4 * j), sv(0, 4 * j + 1));
  #pragma unroll
          for (int kb = 0; kb < T::NKB; ++kb)
  #pragma unroll
            for (int r = 0; r < 16; ++r) {
              if (kb == 0 && (r & 3) < 2) continue;
              mq[r >> 2] = fmaxf(mq[r >> 2], sv(kb, r));
            }
          float mx = fmaxf(fmaxf(mq[0], mq[1]), fmaxf(mq[2], mq[3]));
          {  // max with lane l ^ 32 (the same row) on the VALU
            float a = mx, bb = mx;
            // inline asm: the compiler folds a max of the builtin's two results away
            asm volatile("s_nop 1\n\tv_permlane32_swap_b32 %0, %1" : "+v"(a), "+v"(bb));
            mx = fmaxf(a, bb);
          }
          if (POS_SCALE) mx *= p.sl2;
          // only the rows that need it (either half of the row) raise their
          // maximum; the others keep it (alpha = 1, the same exponentials), so
          // a row's arithmetic does not depend on the other rows of its wave
          float na = need ? 1.f : 0.f, nb = na;
          asm volatile("s_nop 1\n\tv_permlane32_swap_b32 %0, %1" : "+v"(na), "+v"(nb));
          const float m_new = fmaxf(na, nb) > 0.f ? fmaxf(m_run, mx) : m_run;
          const float alpha = (m_new == kNegInf) ? 1.f : fast_exp2(m_run - m_new);
          l_run *= alpha;
  #pragma unroll
          for (int db = 0; db < T::NDB; ++db)
  #pragma unroll
            for (int r = 0; r < 16; ++r) acc[db][r] *= alpha;
          m_run = m_new;
          ls = exp_tile(m_run == kNegInf ? 0.f : m_run);  // row with nothing visible yet
        }
        l_run += ls;
      } else {
  #pragma unroll
        for (int kc = 0; kc < T::VC; ++kc) pk[kc] = u32x4{};
      }
      // the first LA score operands of M(k+1): K(k+1) is complete (see the
      // load schedule) and its slot is not reloaded before M(k+2)
  #pragma unroll
      for (int j = 0; j < NPRE; ++j) kpre[j] = kfrag((decltype(U)::value + 1) % S, j);
      if (group_b) wait_vm<2 * T::LPW * (S - 3)>();
    };

    // prologue: K(0..S-2) and V(0..S-3) in LDS before the first barrier
    unrolled_while<0, S - 1>([&](auto T_) { issue_k(T_); return true; });
    unrolled_while<0, S - 2>([&](auto T_) { issue_v(T_); return true; });
    if constexpr (PAGED) {  // M(0) loads K tile S-1 and V tile S-2
      id_k = lookup(kt - 1);
      id_next = lookup(kt);
      paged_advance();
    }
    wait_vm<0>();  // also completes the Q loads, once, outside the loop
  #pragma unroll
    for (int c = 0; c < T::KC; ++c) asm volatile("" ::"v"(qf[c]));
    lds_barrier();
    if (group_b) lds_barrier();  // B starts one slot behind A
  #pragma unroll
    for (int j = 0; j < NPRE; ++j) kpre[j] = kfrag(0, j);
    // The matrix phase runs at a raised wave priority: the vector phase of
    // the other wave on the SIMD (the older one, for group B) otherwise wins
    // the issue arbitration over its MFMAs.
    auto step = [&](auto U, auto FIRST, int k) __attribute__((always_inline)) {
      int vcase;
      __builtin_amdgcn_s_setprio(1);
      m_phase(U, FIRST, k, vcase);
      lds_barrier();
      __builtin_amdgcn_s_setprio(0);
      v_phase(U, k, vcase);
      lds_barrier_reads_in_flight();
      return k < n_tiles;
    };
    // M(0) has no P V half (there is no tile before tile 0); then S tiles per
    // trip from k = 1, so that every LDS slot index is a compile-time
    // constant; the last step (k = n_tiles) only finishes P V of the last tile
    if (step(integral_constant<int, 0>{}, std::true_type{}, 0)) {
      for (int k0 = 1;; k0 += S) {
        const bool more = unrolled_while<0, S>([&](auto I) {
          constexpr int u = (decltype(I)::value + 1) % S;
          return step(integral_constant<int, u>{}, std::false_type{}, k0 + decltype(I)::value);
        });
        if (!more) break;
      }
    }
    if (!group_b) lds_barrier();  // A's extra barrier matches B's first one
    wait_vm<0>();  // loads past the last tile still land in LDS: drain them
    if (PAGED && bad) s_bad = 1;
    // every wave's loads have landed before the next item's loads start
    __syncthreads();
    if constexpr (PAGED) bad = s_bad != 0;

    // epilogue: O = acc / l (bf16, RNE); LSE = (m + log2 l) ln 2
    float la = l_run, lb = l_run;
    asm volatile("s_nop 1\n\tv_permlane32_swap_b32 %0, %1" : "+v"(la), "+v"(lb));
    const float l_tot = la + lb;
    float inv = l_tot > 0.f ? 1.f / l_tot : 0.f;
    if (PAGED && bad) inv = __builtin_nanf("");  // O and LSE of the whole item are NaN
    if (PAGED && split) {
      // this chunk's normalised O in fp32 and its LSE, for the merge kernel
      const int row = qw0 + n;  // row of the sequence; row - i0 is its row in the tile
      const int64_t prow = ((int64_t)(h * p.vtiles + slot) * p.chunks + chunk) * kBM + (row - i0);
      if (row < Nq) {
  #pragma unroll
        for (int db = 0; db < T::NDB; ++db)
  #pragma unroll
          for (int r4 = 0; r4 < 4; ++r4) {
            f32x4 w;
            w[0] = acc[db][r4 * 4 + 0] * inv;
            w[1] = acc[db][r4 * 4 + 1] * inv;
            w[2] = acc[db][r4 * 4 + 2] * inv;
            w[3] = acc[db][r4 * 4 + 3] * inv;
            *reinterpret_cast<f32x4*>(p.part_o + prow * D + db * 32 + r4 * 8 + g * 4) = w;
          }
        if (g == 0)
          p.part_lse[prow] = bad ? __builtin_nanf("")
                             : l_tot > 0.f ? (m_run + fast_log2(l_tot)) * kLn2 : kNegInf;
      }
    } else {
      // O leaves through LDS as whole rows (rather than as 8-byte pieces
      // scattered over 32 rows), feature half by feature half, in the slots
      // that the next item's prologue does not load: K slot S-1 (waves 0-3)
      // and V slot S-1 (waves 4-7), 32 rows x D/2 features per wave.  The
      // next item's first barrier comes before its M(0) loads K slot S-1.
      // The 16-byte pieces of a staged half row are XOR-swizzled by (row / RB)
      // so that a write of all 64 lanes spreads over the 64 banks.
      constexpr int HB = T::ROWB / 2;     // bytes of a half row
      constexpr int HP = HB / 16;         // its 16-byte pieces
      constexpr int RB = 256 / HB;        // half rows per 256 bytes (all banks)
      constexpr int RPI = 64 / HP;        // half rows per read instruction
      static_assert(kWaves / 2 * kRowsPerWave * HB == T::TILEB, "a slot stages four waves");
      const uint32_t sbase = ((group_b ? S : 0) + S - 1) * T::TILEB +
                             (wave & (kWaves / 2 - 1)) * kRowsPerWave * HB;
      const int rr = lane / HP, cc = lane % HP;
  #pragma unroll
      for (int half = 0; half < 2; ++half) {
  #pragma unroll
        for (int dl = 0; dl < T::NDB / 2; ++dl)
  #pragma unroll
          for (int r4 = 0; r4 < 4; ++r4) {
            const int db = half * (T::NDB / 2) + dl;
            const int piece = (dl * 4 + r4) ^ ((n / RB) & (HP - 1));
            u32x2 w;
            w[0] = pack_bf16x2(acc[db][r4 * 4 + 0] * inv, acc[db][r4 * 4 + 1] * inv);
            w[1] = pack_bf16x2(acc[db][r4 * 4 + 2] * inv, acc[db][r4 * 4 + 3] * inv);
            *reinterpret_cast<__attribute__((address_space(3))) u32x2*>(lds + sbase + n * HB + piece * 16 + g * 8) = w;
          }
        // this wave's own region: its LDS accesses complete in order
  #pragma unroll
        for (int i = 0; i < kRowsPerWave / RPI; ++i) {
          const int r = i * RPI + rr;
          const u32x4 w = *reinterpret_cast<const __attribute__((address_space(3))) u32x4*>(
              lds + sbase + r * HB + ((cc ^ ((r / RB) & (HP - 1))) * 16));
          if (qw0 + r < Nq && qw0 + r >= 0)
            *reinterpret_cast<u32x4*>(p.o + (q_tok0 + qw0 + r) * q_row + (int64_t)h * D + half * (D / 2) + 8 * cc) = w;
        }
      }
      const int row = qw0 + n;
      if (row < Nq && row >= 0 && p.lse != nullptr && g == 0)
        p.lse[lse0 + row] = (PAGED && bad) ? __builtin_nanf("")
                            : l_tot > 0.f ? (m_run + fast_log2(l_tot)) * kLn2 : kNegInf;
    }
  }
  if (tid == 0) s_unit = first + grabbed;
  __syncthreads();
  unit = s_unit;
  }
}

// Paged chunked prefill, second pass: rows of items done in several key
// chunks merge the chunks' (O_c, LSE_c): M = max LSE_c, w_c = exp(LSE_c - M),
// O = sum w_c O_c / sum w_c, LSE = M + ln sum w_c (the exact merge of partial
// softmax states), taken in one pass: the running (m, sum, O) of a row is
// rescaled whenever a chunk raises its maximum, so a row's chunks are read in
// one round of loads.  One work group per (schedule slot, query head); a wave
// takes 8 (D = 128) or 16 (D = 64) rows at a time, 4 features per lane, with
// the loads of all their chunks (up to 4 at a time) in flight together; the
// partials are read once, with non-temporal loads.  A NaN partial (a block the first pass could
// not read) gives NaN.
template <int D>
__global__ __launch_bounds__(256) void prefill_merge_kernel(const Params p) {
  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
  const int slot = blockIdx.x, h = blockIdx.y;
  const int b = find_seq<kBM>(p.cu_q, p.n_seqs, p.total_q, slot, lane);
  const int q0 = clampi(p.cu_q[b], 0, p.total_q);
  const int Nq = clampi(p.cu_q[b + 1], q0, p.total_q) - q0;
  const int len = p.seq_lens[b];
  if (len < 0 || len > p.max_blocks * kBlockTokens) return;  // written as NaN by the first pass
  const int off = slot - (q0 / kBM + b);
  const int ntl = (Nq + kBM - 1) / kBM;
  if (off < 0 || off >= ntl) return;
  const int qt = ntl - 1 - off;
  const TileRange tr = tile_range(qt * kBM, Nq, len, 1, p.window);
  if (tr.n_tiles == 0) return;
  const int c0 = tr.t_begin / p.chunk_tiles;
  const int c1 = (tr.t_begin + tr.n_tiles - 1) / p.chunk_tiles;
  if (c1 == c0) return;  // written directly by the first pass
  // lanes along the features, 4 per lane (16-byte loads): LPR lanes per
  // row, RPI rows per load instruction, R rows of a wave in flight together
  constexpr int LPR = D / 4;
  constexpr int RPI = 64 / LPR;
  constexpr int RI = 4;       // load instructions per chunk
  constexpr int R = RI * RPI;
  constexpr int CG = 4;       // chunks whose loads are issued together
  typedef float f4 __attribute__((ext_vector_type(4)));
  const int sub = lane % LPR, rsub = lane / LPR;
  const int64_t base = (int64_t)(h * p.vtiles + slot) * p.chunks * kBM;
  const int64_t q_row = (int64_t)p.Hq * D;
  const int nrows = min(kBM, Nq - qt * kBM);
  for (int r0 = wave * R; r0 < nrows; r0 += 4 * R) {
    float m[RI], sum[RI];
    f4 o[RI];
    bool nan[RI];
  #pragma unroll
    for (int i = 0; i < RI; ++i) {
      m[i] = kNegInf;
      sum[i] = 0.f;
      o[i] = f4{};
      nan[i] = false;
    }
    for (int cb = c0; cb <= c1; cb += CG) {
      float l[RI][CG];
      f4 v[RI][CG];
  #pragma unroll
      for (int i = 0; i < RI; ++i)
  #pragma unroll
        for (int j = 0; j < CG; ++j) {
          const int r = r0 + i * RPI + rsub;
          const bool ok = cb + j <= c1 && r < nrows;
          const int64_t pr = base + (int64_t)(cb + j) * kBM + r;
          l[i][j] = ok ? __builtin_nontemporal_load(p.part_lse + pr) : kNegInf;
          v[i][j] = ok ? __builtin_nontemporal_load(reinterpret_cast<const f4*>(p.part_o + pr * D + sub * 4))
                       : f4{};
        }
  #pragma unroll
      for (int i = 0; i < RI; ++i)
  #pragma unroll
        for (int j = 0; j < CG; ++j) {
          const float lj = l[i][j];
          nan[i] |= lj != lj;
          const float mn = fmaxf(m[i], lj);  // fmaxf passes over a NaN
          const float a = m[i] == kNegInf ? 0.f : fast_exp2((m[i] - mn) * kLog2e);
          const float w = !(lj > kNegInf) ? 0.f : fast_exp2((lj - mn) * kLog2e);
          sum[i] = sum[i] * a + w;
          o[i] = o[i] * a + v[i][j] * w;
          m[i] = mn;
        }
    }
  #pragma unroll
    for (int i = 0; i < RI; ++i) {
      const int r = r0 + i * RPI + rsub;
      if (r >= nrows) continue;
      const float inv = nan[i] ? __builtin_nanf("") : sum[i] > 0.f ? 1.f / sum[i] : 0.f;
      const int row = qt * kBM + r;
      u32x2 w;
      w[0] = pack_bf16x2(o[i][0] * inv, o[i][1] * inv);
      w[1] = pack_bf16x2(o[i][2] * inv, o[i][3] * inv);
      *reinterpret_cast<u32x2*>(p.o + ((int64_t)q0 + row) * q_row + (int64_t)h * D + sub * 4) = w;
      if (sub == 0 && p.lse != nullptr)
        p.lse[(int64_t)h * p.total_q + q0 + row] =
            nan[i] ? __builtin_nanf("") : sum[i] > 0.f ? m[i] + fast_log2(sum[i]) * kLn2 : kNegInf;
    }
  }
}

}  // namespace

long long fwd_bf16_grid(int B, int Hq, int Nq) {
  return (long long)B * Hq * ((Nq + kBM - 1) / kBM);
}

namespace {

// Host side of the scheduling counters, per device: the tag counter, the
// next eager and graph slots, and for each eager slot an event recorded after
// the last launch that used it.
constexpr int kMaxDevices = 64;
struct SchedState {
  std::mutex mu;
  unsigned tag = 0;
  int next_eager = 0, next_graph = 0;
  int eager_slots = kEagerSlots;  // slots in turn (tests may lower it)
  hipEvent_t ev[kEagerSlots] = {};
  bool recorded[kEagerSlots] = {};
};
SchedState g_state[kMaxDevices];

// one persistent work group per CU (the LDS ring admits one per CU)
template <int MODE>
hipError_t launch(Params& p, int d, float scale, long long units, hipStream_t stream) {
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
  hipStreamCaptureStatus cap = hipStreamCaptureStatusNone;
  e = hipStreamIsCapturing(stream, &cap);
  if (e != hipSuccess) return e;
  SchedState& st = g_state[dev];
  std::lock_guard<std::mutex> lock(st.mu);
  if (++st.tag == 0) ++st.tag;  // 0 is no launch's tag
  p.tag = st.tag;
  int eager = -1;
  if (cap != hipStreamCaptureStatusNone) {
    // a slot of its own: replays of this graph reuse it, set up afresh each time
    p.slot = kEagerSlots + st.next_graph;
    st.next_graph = (st.next_graph + 1) % kGraphSlots;
  } else {
    eager = st.next_eager % st.eager_slots;
    st.next_eager = (eager + 1) % st.eager_slots;
    p.slot = eager;
    if (st.recorded[eager]) {
      // the slot's previous launch may still run (on any stream): wait for it
      e = hipEventQuery(st.ev[eager]);
      if (e == hipErrorNotReady) e = hipStreamWaitEvent(stream, st.ev[eager], 0);
      if (e != hipSuccess) return e;
    } else if (st.ev[eager] == nullptr) {
      e = hipEventCreateWithFlags(&st.ev[eager], hipEventDisableTiming);
      if (e != hipSuccess) return e;
    }
  }
  hipLaunchKernelGGL(sched_reset_kernel, dim3(1), dim3(64), 0, stream, p.slot, p.tag);
  const int cus = device_cus();
  const dim3 grid(units < cus ? (int)units : cus), block(kThreads);
  const bool pos = scale > 0.f;
  if (d == 128) {
    if (pos)
      hipLaunchKernelGGL((fwd_bf16_kernel<128, true, MODE>), grid, block, 0, stream, p);
    else
      hipLaunchKernelGGL((fwd_bf16_kernel<128, false, MODE>), grid, block, 0, stream, p);
  } else {
    if (pos)
      hipLaunchKernelGGL((fwd_bf16_kernel<64, true, MODE>), grid, block, 0, stream, p);
    else
      hipLaunchKernelGGL((fwd_bf16_kernel<64, false, MODE>), grid, block, 0, stream, p);
  }
  e = hipGetLastError();
  if (e == hipSuccess && eager >= 0) {
    e = hipEventRecord(st.ev[eager], stream);
    st.recorded[eager] = e == hipSuccess;
  }
  return e;
}

}  // namespace

int set_fwd_sched_slots(int n) {
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return -1;
  SchedState& st = g_state[dev];
  std::lock_guard<std::mutex> lock(st.mu);
  const int prev = st.eager_slots;
  if (n >= 1 && n <= kEagerSlots) st.eager_slots = n;
  return prev;
}

hipError_t launch_fwd_bf16(const FwdArgs& a, hipStream_t stream) {
  Params p{};
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
  // grouped heads: an item holds kBM / gpack positions of gpack query heads
  // that share a KV head, gpack the largest of 8, 4, 2 dividing the group
  // (never more work units than fwd_bf16_grid counts)
  p.gpack = p.group % 8 == 0 ? 8 : p.group % 4 == 0 ? 4 : p.group % 2 == 0 ? 2 : 1;
  const int rows = kBM / p.gpack;
  p.n_qtiles = (a.Nq + rows - 1) / rows;
  p.total = (int)((long long)a.B * (a.Hq / p.gpack) * p.n_qtiles);
  p.sl2 = a.scale * kLog2e;
  if (p.total == 0) return hipSuccess;
  // pair query tiles when there are enough pairs to fill the CUs
  const long long pairs = (long long)(p.total / p.n_qtiles) * ((p.n_qtiles + 1) / 2);
  p.pairing = pairs >= device_cus() ? 1 : 0;
  return launch<kDense>(p, a.d, a.scale, p.pairing ? pairs : p.total, stream);
}

long long fwd_bf16_varlen_grid(int n_seqs, int Hq, int total_q) {
  return (long long)Hq * (total_q / kBM + n_seqs);
}

hipError_t launch_fwd_bf16_varlen(const FwdVarlenArgs& a, hipStream_t stream) {
  Params p{};
  p.q = static_cast<const uint16_t*>(a.q);
  p.k = static_cast<const uint16_t*>(a.k);
  p.v = static_cast<const uint16_t*>(a.v);
  p.o = static_cast<uint16_t*>(a.out);
  p.lse = a.lse;
  p.Hq = a.Hq;
  p.Hkv = a.Hkv;
  p.group = a.Hq / a.Hkv;
  p.causal = a.causal;
  p.window = a.window;
  p.sl2 = a.scale * kLog2e;
  p.cu_q = a.cu_seqlens_q;
  p.cu_k = a.cu_seqlens_k;
  p.n_seqs = a.n_seqs;
  p.total_q = a.total_q;
  p.total_k = a.total_k;
  p.vtiles = a.total_q / kBM + a.n_seqs;
  p.n_qtiles = 1;
  p.pairing = 0;
  p.total = (int)fwd_bf16_varlen_grid(a.n_seqs, a.Hq, a.total_q);
  if (a.n_seqs == 0 || a.total_q == 0) return hipSuccess;
  return launch<kVarlen>(p, a.d, a.scale, p.total, stream);
}

hipError_t launch_prefill_paged(const PrefillPagedArgs& a, hipStream_t stream) {
  Params p{};
  p.q = static_cast<const uint16_t*>(a.q);
  p.k = static_cast<const uint16_t*>(a.kcache);
  p.v = static_cast<const uint16_t*>(a.vcache);
  p.o = static_cast<uint16_t*>(a.out);
  p.lse = a.lse;
  p.Hq = a.Hq;
  p.Hkv = a.Hkv;
  p.group = a.Hq / a.Hkv;
  p.causal = 1;
  p.window = a.window;
  p.sl2 = a.scale * kLog2e;
  p.cu_q = a.cu_seqlens_q;
  p.table = a.block_table;
  p.seq_lens = a.seq_lens;
  p.max_blocks = a.max_blocks_per_seq;
  p.num_blocks = a.num_blocks;
  p.n_seqs = a.n_seqs;
  p.total_q = a.total_q;
  p.vtiles = a.total_q / kBM + a.n_seqs;
  p.n_qtiles = 1;
  p.pairing = 0;
  p.chunk_tiles = kChunkTiles;
  p.chunks = prefill_paged_chunks(a.max_blocks_per_seq);
  char* ws = static_cast<char*>(a.workspace);
  p.part_o = reinterpret_cast<float*>(ws);
  p.part_lse = reinterpret_cast<float*>(
      ws + prefill_paged_part_o_bytes(a.n_seqs, a.Hq, a.total_q, a.d, a.max_blocks_per_seq));
  p.total = (int)prefill_paged_grid(a.n_seqs, a.Hq, a.total_q, a.max_blocks_per_seq);
  if (a.n_seqs == 0 || a.total_q == 0) return hipSuccess;
  const hipError_t e = launch<kPaged>(p, a.d, a.scale, p.total, stream);
  if (e != hipSuccess || p.chunks == 1) return e;
  const dim3 grid(p.vtiles, a.Hq);
  if (a.d == 128)
    hipLaunchKernelGGL(prefill_merge_kernel<128>, grid, dim3(256), 0, stream, p);
  else
    hipLaunchKernelGGL(prefill_merge_kernel<64>, grid, dim3(256), 0, stream, p);
  return hipGetLastError();
}

int prefill_paged_chunks(int max_blocks_per_seq) {
  const long long tiles = ((long long)max_blocks_per_seq * kBlockTokens + 63) / 64;
  return (int)((tiles + kChunkTiles - 1) / kChunkTiles);
}

long long prefill_paged_grid(int n_seqs, int Hq, int total_q, int max_blocks_per_seq) {
  return fwd_bf16_varlen_grid(n_seqs, Hq, total_q) * prefill_paged_chunks(max_blocks_per_seq);
}

size_t prefill_paged_part_o_bytes(int n_seqs, int Hq, int total_q, int d, int max_blocks_per_seq) {
  const int c = prefill_paged_chunks(max_blocks_per_seq);
  if (c <= 1) return 0;
  const size_t rows = (size_t)fwd_bf16_varlen_grid(n_seqs, Hq, total_q) * c * kBM;
  return (rows * d * sizeof(float) + 255) / 256 * 256;
}

size_t prefill_paged_workspace_bytes(int n_seqs, int Hq, int total_q, int d,
                                     int max_blocks_per_seq) {
  const int c = prefill_paged_chunks(max_blocks_per_seq);
  if (c <= 1) return 0;
  const size_t rows = (size_t)fwd_bf16_varlen_grid(n_seqs, Hq, total_q) * c * kBM;
  return prefill_paged_part_o_bytes(n_seqs, Hq, total_q, d, max_blocks_per_seq) +
         (rows * sizeof(float) + 255) / 256 * 256;
}

}  // namespace attn
