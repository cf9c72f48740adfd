/*
 * attn.h — C ABI of the MI355X (gfx950) exact softmax attention library.
 *
 * Two operations, both exact (up to floating-point rounding order) scaled
 * dot-product attention O = softmax(scale * Q K^T + mask) V:
 *
 *   attn_fwd / attn_fwd_f32  prefill / training forward over dense Q, K, V,
 *                            tiled and fused with an online softmax so the
 *                            score matrix never reaches device memory, with
 *                            causal and sliding-window masks and grouped
 *                            K/V heads (MHA, GQA, MQA);
 *   attn_fwd_varlen          the same forward over packed sequences of
 *                            different lengths (no padding), each attending
 *                            only within itself;
 *   attn_decode_paged        one query per sequence over a block-paged KV
 *                            cache, split along the keys with a final merge;
 *   attn_prefill_paged       several new tokens per sequence (a prefill
 *                            chunk) over the same paged cache;
 *   attn_bwd                 the gradients of attn_fwd (bf16), recomputing
 *                            the probabilities from the saved log-sum-exp;
 *   attn_bwd_varlen          the gradients of attn_fwd_varlen;
 *   attn_merge               the exact merge of two partial results over
 *                            disjoint key sets (the combine step of attention
 *                            split along the keys, e.g. across devices).
 *
 * Sources (pages; section names as printed):
 *   - "Attention Is O(n^2): FlashAttention vs Linear Attention", "Why
 *     Attention Is O(n^2)" (the definition) and "FlashAttention - Same
 *     FLOPs, Linear Memory" (query-block / key-block loop with a running
 *     maximum and sum, final normalisation, float32 log-sum-exp kept for the
 *     backward pass).
 *   - "Ch. 3: MHA Limitations, MQA, GQA, and FlashAttention", 3.3 (query head
 *     i reads K/V head i / (Hq / Hkv); Hq must be a multiple of Hkv), 3.5
 *     (merging partial softmax statistics across key tiles), 3.1 (decode: a
 *     new query reads the cached K/V, its own K/V appended first).
 *   - "Modern Attention: MQA, GQA, FlashAttention, Sliding Window and RoPE",
 *     3 (online softmax) and 4 (a token sees the last W tokens).
 *   - "Inference Engineering", 2.5 "Optimizing Attention" (PagedAttention:
 *     the cache is split into blocks reached through a lookup table).
 *   - "How to Reduce Attention Computation Cost in LLM Training",
 *     "FlashAttention Is Table Stakes" (fused call on (B, N, H, d) bf16;
 *     packed sequence boundaries need variable-length kernels), the
 *     comparison table and FAQ (sequence packing).
 *
 * Conventions shared by every entry point
 *   - All tensor pointers are DEVICE pointers owned by the caller; nothing is
 *     retained after the call returns.  Tensors are dense, row-major, with no
 *     padding.  Outputs must not alias inputs (attn_merge alone allows an
 *     in-place merge).
 *   - Every call is asynchronous on `stream` (a hipStream_t passed as void*;
 *     NULL means the default stream).  The library never synchronises and
 *     never allocates device memory.
 *   - Arguments are validated on the host before any HIP call; a negative
 *     status is returned and nothing is launched.  Values that live in device
 *     memory (sequence lengths, block ids) are checked by the kernels, which
 *     write NaN for a sequence they cannot read safely and never read out of
 *     bounds.
 *   - Masks (reading of the pages where they are silent):
 *       causal:  query row i sits at absolute position i + (Nk - Nq)
 *                ("bottom-right"), and sees keys j <= that position;
 *       window:  W > 0 keeps the last W keys up to and including the query's
 *                own position (position - j < W); it requires causal.
 *     A query row that sees no key gets O = 0 and LSE = -inf.
 *   - LSE is the natural logarithm of sum_j exp(scale * q.k_j) over the
 *     visible keys, in float32.
 *   - `scale` is used as given (callers normally pass 1/sqrt(d)).
 *   - The library is thread-safe.  Its state is a per-device cache of the
 *     compute-unit count, filled on first use, and the scheduling counters of
 *     the bf16 forward kernels (attn_fwd, attn_fwd_varlen, attn_prefill_paged):
 *     each launch takes a fresh tag and a slot of counters in device memory,
 *     and is preceded on its stream by a one-wave kernel that sets the slot up.
 *     Slot use is exclusive: 256 slots are taken in turn, and a launch whose
 *     slot's previous launch has not finished first waits for it on its stream
 *     (an event the library records after each launch), so any number of
 *     launches may be in flight on any streams.
 *   - Graph capture: a forward call made while its stream is capturing
 *     records two kernel launches (the counter set-up and the kernel) and
 *     takes a slot of its own, out of 4096 reserved for captured calls and
 *     reused in turn; no event is recorded.  Every replay sets the slot up
 *     again, so replays in turn are correct.  Replays of one captured call
 *     must not overlap each other (they also write the same outputs), nor may
 *     replays of calls captured 4096 captures apart.
 */
#ifndef ATTN_MI355X_ATTN_H
#define ATTN_MI355X_ATTN_H

#include <stddef.h>

#ifdef __cplusplus
extern "C" {
#endif

/* Status codes. */
enum {
  ATTN_OK = 0,
  ATTN_E_NULL = -1,      /* a required pointer is NULL                          */
  ATTN_E_SHAPE = -2,     /* bad size: negative, Hq % Hkv != 0, causal with      */
                         /* Nq > Nk, unsupported block size, grid too large     */
  ATTN_E_HEADDIM = -3,   /* head dimension d not in {64, 128}                   */
  ATTN_E_MASK = -4,      /* window > 0 without causal                           */
  ATTN_E_WORKSPACE = -5, /* workspace NULL or smaller than the query says       */
  ATTN_E_LAUNCH = -6     /* the HIP runtime reported an error at launch         */
};

/*
 * Prefill / training forward, bf16 in and out, float32 accumulation.
 *
 * Defines: O = softmax(scale * Q K^T + mask) V per (batch, query head)
 * ("Attention Is O(n^2): FlashAttention vs Linear Attention", "Why Attention
 * Is O(n^2)"), computed by the query-block / key-block loop of that page's
 * "FlashAttention - Same FLOPs, Linear Memory" (running maximum and sum,
 * rescale, final division; the float32 log-sum-exp is kept for the backward
 * pass); grouped K/V heads as in "Ch. 3: MHA Limitations, MQA, GQA, and
 * FlashAttention", 3.3; the sliding window of "Modern Attention: MQA, GQA,
 * FlashAttention, Sliding Window and RoPE", 4; the (B, N, H, d) bf16 layout of
 * the fused call in "How to Reduce Attention Computation Cost in LLM
 * Training", "FlashAttention Is Table Stakes Now".
 *
 *   q    [B, Nq, Hq, d]   bf16
 *   k, v [B, Nk, Hkv, d]  bf16
 *   out  [B, Nq, Hq, d]   bf16 (rounded to nearest even)
 *   lse  [B, Hq, Nq]      float32, or NULL to skip it
 *
 * Sizes: B, Nq, Nk >= 0 (B == 0 or Nq == 0 is a no-op; Nk == 0 gives O = 0,
 * LSE = -inf); Hq, Hkv >= 1 with Hq % Hkv == 0; d in {64, 128}; Hkv * d <=
 * 4194304 (key tiles are addressed with 32-bit byte offsets).  Pointers of
 * tensors with no elements may be NULL; the others must not be (ATTN_E_NULL).
 * causal: 0 or 1; causal requires Nq <= Nk.  window: <= 0 for none, else the
 * number of keys kept (requires causal).
 */
int attn_fwd(const void* q, const void* k, const void* v, void* out, float* lse,
             int B, int Hq, int Hkv, int Nq, int Nk, int d,
             int causal, int window, float scale, void* stream);

/*
 * The same operation on float32 q, k, v and out, with float32 products and
 * accumulation throughout (no reduced-precision matrix formats).  Parameters
 * and rules are those of attn_fwd.  Defines the same result: the definition
 * in "Attention Is O(n^2): FlashAttention vs Linear Attention", "Why
 * Attention Is O(n^2)", whose "Wall-Clock Impact of Tiling" runs it at d = 64
 * with float inputs; the online softmax of "Modern Attention: MQA, GQA,
 * FlashAttention, Sliding Window and RoPE", 3 (its worked example is one of
 * this entry point's tests).
 */
int attn_fwd_f32(const float* q, const float* k, const float* v, float* out, float* lse,
                 int B, int Hq, int Hkv, int Nq, int Nk, int d,
                 int causal, int window, float scale, void* stream);

/*
 * Forward over packed sequences ("How to Reduce Attention Computation Cost in
 * LLM Training": packed sequence boundaries need variable-length kernels,
 * section "FlashAttention Is Table Stakes Now"; packing many short sequences
 * instead of padding them, the comparison table and the FAQ).  bf16 in and
 * out, float32 accumulation, the kernel of attn_fwd.
 *
 *   q, out        [total_q, Hq, d]   bf16: the sequences' query rows back to back
 *   k, v          [total_k, Hkv, d]  bf16: their key rows back to back
 *   cu_seqlens_q  [num_seqs + 1] int32, DEVICE memory: sequence s owns query
 *                 rows cu_seqlens_q[s] .. cu_seqlens_q[s+1]-1
 *   cu_seqlens_k  [num_seqs + 1] int32, DEVICE memory: likewise for key rows
 *   lse           [Hq, total_q] float32, or NULL to skip it
 *
 * Each sequence attends only to its own keys; causal alignment and the
 * window apply within the sequence (its query row i sits at i + nk - nq).
 * A sequence may have more queries than keys: under causal its first rows
 * see no key and get O = 0, LSE = -inf.  Rows of q outside every sequence
 * are not written.
 *
 * The cu arrays must be nondecreasing with entries in [0, total]; values
 * outside are clamped into range as read (no access leaves the tensors) but
 * the results are then unspecified.  The host never reads them.
 *
 * Sizes: num_seqs, total_q, total_k >= 0 (num_seqs == 0 or total_q == 0 is
 * a no-op); Hq, Hkv, d, causal and window as for attn_fwd;
 * Hq * (total_q / 256 + num_seqs) <= INT_MAX (ATTN_E_SHAPE).
 */
int attn_fwd_varlen(const void* q, const void* k, const void* v, void* out, float* lse,
                    const int* cu_seqlens_q, const int* cu_seqlens_k, int num_seqs,
                    int total_q, int total_k, int Hq, int Hkv, int d,
                    int causal, int window, float scale, void* stream);

/*
 * Bytes of device workspace attn_decode_paged needs for these sizes
 * (0 for invalid sizes).  Pure host function; no HIP call.
 */
size_t attn_decode_paged_workspace_size(int B, int Hq, int d, int block_size,
                                        int max_blocks_per_seq);

/*
 * Single-query decode over a block-paged KV cache.
 *
 * Defines: for each sequence, the attention of its newest token's query over
 * every cached key and value of that sequence, its own K/V included ("Ch. 3:
 * MHA Limitations, MQA, GQA, and FlashAttention", 3.1: each new query reads
 * the historical K/V, its own appended first); the cache is split into
 * fixed-size blocks reached through a lookup table ("Inference Engineering",
 * 2.5 "Optimizing Attention", PagedAttention); the keys are processed in
 * pieces whose partial softmax states are merged exactly ("Ch. 3", 3.5).
 *
 *   q            [B, Hq, d] bf16: the query of the token at position
 *                seq_lens[b] - 1, whose own K/V are already in the cache
 *   kcache,
 *   vcache       [num_blocks, block_size, Hkv, d] bf16
 *   block_table  [B, max_blocks_per_seq] int32: logical token t of sequence b
 *                is slot t % block_size of block block_table[b][t / block_size];
 *                entries past ceil(seq_lens[b] / block_size) are ignored
 *   seq_lens     [B] int32, cached tokens per sequence (device memory)
 *   out          [B, Hq, d] bf16
 *   lse          [B, Hq] float32, or NULL
 *   window       <= 0: attend every cached token; else the last `window`
 *   workspace    device scratch of at least
 *                attn_decode_paged_workspace_size(...) bytes, owned by the
 *                caller; its contents on entry do not matter
 *
 * block_size must be 16; d in {64, 128}; Hq % Hkv == 0; B <= 65535, Hq <= 65535
 * and B * max_blocks_per_seq <= INT_MAX (ATTN_E_SHAPE otherwise).  A sequence with
 * seq_len == 0 gets O = 0, LSE = -inf.  A sequence whose length is negative or
 * exceeds max_blocks_per_seq * block_size, or whose table names a block
 * outside [0, num_blocks), gets NaN in out and lse.  Only the used slots of the
 * cache are read; unused blocks and tail slots may hold anything (NaN too).
 */
int attn_decode_paged(const void* q, const void* kcache, const void* vcache,
                      const int* block_table, const int* seq_lens, void* out, float* lse,
                      int B, int Hq, int Hkv, int d, int block_size, int max_blocks_per_seq,
                      int num_blocks, int window, float scale,
                      void* workspace, size_t workspace_bytes, void* stream);

/*
 * attn_decode_paged without a workspace argument, for callers that cannot
 * allocate device memory: code under HIP graph capture, tight serving loops,
 * harnesses that forbid allocation.  It allocates nothing and calls no
 * allocating routine: the partial results live in the library's own device
 * array of 16 MiB per GPU (set up when the library's code is loaded on that
 * GPU and kept until the process ends).  The first call on each device looks
 * up the array's address (a HIP symbol query, no allocation).  Arguments,
 * layouts and results are those of attn_decode_paged (the same kernels; the
 * outputs are equal bit for bit); ATTN_E_WORKSPACE when
 * attn_decode_paged_workspace_size(B, Hq, d, block_size, max_blocks_per_seq)
 * exceeds 16 MiB (e.g. B <= 16 with Hq * d <= 4096).  Nothing in the array
 * needs to start at zero.  Every call on one GPU shares that GPU's array:
 * calls that overlap in time on one GPU (different streams or threads) race
 * and must not be made.
 */
int attn_decode_paged_noalloc(const void* q, const void* kcache, const void* vcache,
                              const int* block_table, const int* seq_lens, void* out,
                              float* lse, int B, int Hq, int Hkv, int d, int block_size,
                              int max_blocks_per_seq, int num_blocks, int window, float scale,
                              void* stream);

/*
 * Bytes of device workspace attn_prefill_paged needs for these sizes (0 when
 * no query tile can need more than one key chunk of 8192 keys, i.e.
 * max_blocks_per_seq * block_size <= 8192; 0 for invalid sizes).  Pure host
 * function; no HIP call.
 */
size_t attn_prefill_paged_workspace_size(int num_seqs, int total_q, int Hq, int d,
                                         int block_size, int max_blocks_per_seq);

/*
 * Chunked prefill over a block-paged KV cache ("Ch. 3: MHA Limitations, MQA,
 * GQA, and FlashAttention": 3.1, new tokens attend to the cache after their
 * own K/V are appended; the GQA code of 3.3 notes that a cache needs its own
 * causal handling; "Inference Engineering", 2.5: the cache is split into
 * blocks reached through a lookup table).  The kernel of attn_fwd reading
 * K/V through the table.  A 256-row query tile whose keys span more than one
 * 8192-key chunk is computed chunk by chunk (separate work units, partial
 * results in the workspace) and merged by a second kernel on the same stream
 * ("Ch. 3" 3.5: partial softmax states merge exactly).
 *
 *   q, out        [total_q, Hq, d] bf16: each sequence's new tokens back to back
 *   cu_seqlens_q  [num_seqs + 1] int32 (device): sequence s owns rows
 *                 cu_seqlens_q[s] .. cu_seqlens_q[s+1]-1 (nq_s rows)
 *   kcache,
 *   vcache        [num_blocks, block_size, Hkv, d] bf16, as for attn_decode_paged
 *   block_table   [num_seqs, max_blocks_per_seq] int32 (device)
 *   seq_lens      [num_seqs] int32 (device): cached tokens of sequence s, its
 *                 new tokens included (they are the last nq_s of them)
 *   lse           [Hq, total_q] float32, or NULL
 *   workspace     attn_prefill_paged_workspace_size(...) bytes of device
 *                 memory owned by the caller (may be NULL when that is 0); its
 *                 contents on entry do not matter; calls that share it must
 *                 not overlap
 *
 * Always causal: new row i of sequence s sits at position seq_lens[s] - nq_s
 * + i and sees the cached tokens up to it (the last `window` of them when
 * window > 0).  Rows at negative positions (nq_s > seq_lens[s]) see no key
 * and get O = 0, LSE = -inf.  A sequence whose length is negative or exceeds
 * max_blocks_per_seq * block_size, or whose table names a block outside
 * [0, num_blocks) among its first ceil(seq_lens[s] / block_size) entries
 * (read or not), gets NaN in all its rows.  Nothing outside the pool, those
 * table entries and the given rows is read; rows of q outside every
 * sequence are not written.  The cu
 * array follows the rules of attn_fwd_varlen.
 *
 * block_size must be 16; d in {64, 128}; Hq % Hkv == 0; num_seqs *
 * max_blocks_per_seq <= INT_MAX; Hq * (total_q / 256 + num_seqs) * chunks <=
 * INT_MAX with chunks = ceil(max_blocks_per_seq * 16 / 8192) (ATTN_E_SHAPE
 * otherwise); ATTN_E_WORKSPACE for a missing or short workspace.
 */
int attn_prefill_paged(const void* q, const void* kcache, const void* vcache,
                       const int* block_table, const int* seq_lens, const int* cu_seqlens_q,
                       void* out, float* lse, int num_seqs, int total_q, int Hq, int Hkv, int d,
                       int block_size, int max_blocks_per_seq, int num_blocks, int window,
                       float scale, void* workspace, size_t workspace_bytes, void* stream);

/*
 * Bytes of device workspace attn_bwd needs (two float32 values per query row
 * and head; 0 for invalid sizes).  Pure host function; no HIP call.
 */
size_t attn_bwd_workspace_size(int B, int Hq, int Nq);

/*
 * Backward pass of attn_fwd: the gradients of L = sum(dout * out) with
 * respect to q, k and v, recomputing the probabilities from the saved
 * log-sum-exp instead of storing them ("Ch. 3: MHA Limitations, MQA, GQA,
 * and FlashAttention", 3.5).  With P = exp(scale * q k^T - lse) over the
 * visible keys:
 *   dv = P^T dout,  dS = P * (dout v^T - D) with D_i = sum_c dout_ic out_ic,
 *   dq = scale * dS k,  dk = scale * dS^T q,
 * and a K/V head shared by several query heads receives the sum of their dk
 * and dv.
 *
 *   q, out, dout  [B, Nq, Hq, d] bf16 (out and lse as attn_fwd returned them)
 *   k, v          [B, Nk, Hkv, d] bf16
 *   lse           [B, Hq, Nq] float32 (natural log; -inf for a row without keys)
 *   dq            [B, Nq, Hq, d] bf16 (rounded to nearest even)
 *   dk, dv        [B, Nk, Hkv, d] bf16
 *   workspace     device scratch of at least attn_bwd_workspace_size(B, Hq, Nq)
 *                 bytes, owned by the caller; its contents on entry do not matter
 *
 * Sizes, masks (causal, window, scale) and their rules are those of attn_fwd;
 * B, Hq, Hkv <= 65535 (grid limits).  Every element of dq, dk and dv is
 * written (zero where nothing contributes).  The result does not depend on
 * scheduling: no atomics.
 */
int attn_bwd(const void* q, const void* k, const void* v, const void* out, const void* dout,
             const float* lse, void* dq, void* dk, void* dv,
             int B, int Hq, int Hkv, int Nq, int Nk, int d,
             int causal, int window, float scale,
             void* workspace, size_t workspace_bytes, void* stream);

/* Static, human-readable text for a status code. */
const char* attn_status_str(int status);

/*
 * Testing hook: the number of scheduling-counter slots the bf16 forward
 * launches made outside graph capture take in turn on the current device
 * (1 .. 256, default 256; other values leave it unchanged).  Returns the
 * previous number (-1 if no device is current).  With one slot, every launch
 * waits for the previous one, whatever its stream; results do not change.
 * Host state only; the only HIP call is the current-device query.
 */
int attn_set_fwd_sched_slots(int n);

/*
 * Gradients of attn_fwd_varlen (packed sequences; "How to Reduce Attention
 * Computation Cost in LLM Training" counts packing among the main savings of
 * training, which needs this backward).  The same three kernels as attn_bwd,
 * scheduled over each sequence's 128-row tiles.
 *
 *   q, out, dout, dq  [total_q, Hq, d] bf16;  k, v, dk, dv [total_k, Hkv, d] bf16
 *   lse               [Hq, total_q] float32 from attn_fwd_varlen (required)
 *   cu_seqlens_q/_k   as for attn_fwd_varlen (device int32, num_seqs + 1)
 *   workspace         attn_bwd_workspace_size(1, Hq, total_q) bytes of device memory
 *
 * Each sequence's gradients are those of its own attention (masks and
 * bottom-right alignment within the sequence); a sequence with no query rows
 * gets dK = dV = 0, one with no keys dQ = 0.  Rows outside every sequence are
 * not written.  Sizes and masks as for attn_fwd_varlen, plus Hq <= 65535 and
 * total_q * Hq * d <= 2^40 (ATTN_E_SHAPE); ATTN_E_WORKSPACE for a missing or
 * short workspace.
 */
int attn_bwd_varlen(const void* q, const void* k, const void* v, const void* out,
                    const void* dout, const float* lse, void* dq, void* dk, void* dv,
                    const int* cu_seqlens_q, const int* cu_seqlens_k, int num_seqs,
                    int total_q, int total_k, int Hq, int Hkv, int d, int causal, int window,
                    float scale, void* workspace, size_t workspace_bytes, void* stream);

/*
 * Exact merge of two partial results of the same query rows, each the
 * attention of those rows over one of two disjoint key sets (as attn_fwd
 * writes them): with w = exp(LSE - max(LSE_a, LSE_b)),
 * O = (w_a O_a + w_b O_b) / (w_a + w_b) and LSE = max + ln(w_a + w_b)
 * ("Ch. 3: MHA Limitations, MQA, GQA, and FlashAttention", 3.5: partial
 * softmax states merge exactly after rescaling to a common maximum).  This
 * is the combine step of attention split along the keys, e.g. a device of a
 * ring that attends its queries to one K/V shard at a time ("How to Reduce
 * Attention Computation Cost in LLM Training", ring attention section).
 *
 *   o_a, o_b, out        [B, N, H, d] bf16 (rounded to nearest even)
 *   lse_a, lse_b         [B, H, N] float32; lse_out the same, or NULL
 *
 * out may be o_a and lse_out may be lse_a (an in-place running merge); no
 * other overlap is allowed.  A row with LSE = -inf on both sides gets O = 0,
 * LSE = -inf; a NaN LSE on either side gives NaN.  B, N >= 0, H >= 1, d in
 * {64, 128}, B * N * H * d <= 2^40.
 */
int attn_merge(const void* o_a, const float* lse_a, const void* o_b, const float* lse_b,
               void* out, float* lse_out, int B, int N, int H, int d, void* stream);

#ifdef __cplusplus
}
#endif

#endif /* ATTN_MI355X_ATTN_H */
