// Host-side launch interface between the C ABI (api.cpp) and the kernels.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>

namespace attn {

// Compute units of the current device (looked up once per device).
int device_cus();

struct FwdArgs {
  const void* q;
  const void* k;
  const void* v;
  void* out;
  float* lse;
  int B, Hq, Hkv, Nq, Nk, d;
  int causal, window;
  float scale;
};

// Both assume arguments already validated (d in {64,128}, Hq % Hkv == 0, ...).
hipError_t launch_fwd_bf16(const FwdArgs& a, hipStream_t stream);
hipError_t launch_fwd_f32(const FwdArgs& a, hipStream_t stream);
// Work groups the forward launch uses (for the grid-size check).
long long fwd_bf16_grid(int B, int Hq, int Nq);
long long fwd_f32_grid(int B, int Hq, int Nq);

// Packed sequences: sequence s owns query rows [cu_seqlens_q[s], cu_seqlens_q[s+1])
// of q/out (total_q rows) and key rows [cu_seqlens_k[s], cu_seqlens_k[s+1]) of
// k/v (total_k rows); the cu arrays are device memory of n_seqs + 1 ints.
struct FwdVarlenArgs {
  const void* q;
  const void* k;
  const void* v;
  void* out;
  float* lse;
  const int* cu_seqlens_q;
  const int* cu_seqlens_k;
  int n_seqs, total_q, total_k, Hq, Hkv, d;
  int causal, window;
  float scale;
};

hipError_t launch_fwd_bf16_varlen(const FwdVarlenArgs& a, hipStream_t stream);
// Number of scheduling-counter slots the bf16 forward launches made outside
// graph capture take in turn on the current device (1 .. 256; other values
// leave it unchanged); returns the previous number.
int set_fwd_sched_slots(int n);
// Work units of the packed launch (for the size check).
long long fwd_bf16_varlen_grid(int n_seqs, int Hq, int total_q);

// Chunked prefill over a paged cache: sequence s owns query rows
// [cu_seqlens_q[s], cu_seqlens_q[s+1]) of q/out, the last of its seq_lens[s]
// cached tokens; caches are [num_blocks, 16, Hkv, d].
struct PrefillPagedArgs {
  const void* q;
  const void* kcache;
  const void* vcache;
  const int* block_table;
  const int* seq_lens;
  const int* cu_seqlens_q;
  void* out;
  float* lse;
  int n_seqs, total_q, Hq, Hkv, d, max_blocks_per_seq, num_blocks, window;
  float scale;
  void* workspace;  // prefill_paged_workspace_bytes(...) bytes (none when 0)
};

hipError_t launch_prefill_paged(const PrefillPagedArgs& a, hipStream_t stream);
// Key chunks an item may be split into, work units, and the partial-result
// workspace (fp32 O then LSE per chunk and row; 0 bytes when nothing splits).
int prefill_paged_chunks(int max_blocks_per_seq);
long long prefill_paged_grid(int n_seqs, int Hq, int total_q, int max_blocks_per_seq);
size_t prefill_paged_part_o_bytes(int n_seqs, int Hq, int total_q, int d, int max_blocks_per_seq);
size_t prefill_paged_workspace_bytes(int n_seqs, int Hq, int total_q, int d,
                                     int max_blocks_per_seq);

struct DecodeArgs {
  const void* q;
  const void* kcache;
  const void* vcache;
  const int* block_table;
  const int* seq_lens;
  void* out;
  float* lse;
  int B, Hq, Hkv, d, block_size, max_blocks_per_seq, num_blocks, window;
  float scale;
  void* workspace;
};

struct BwdArgs {
  const void* q;
  const void* k;
  const void* v;
  const void* out;
  const void* dout;
  const float* lse;
  void* dq;
  void* dk;
  void* dv;
  int B, Hq, Hkv, Nq, Nk, d;
  int causal, window;
  float scale;
  void* workspace;
};

size_t bwd_workspace_bytes(int B, int Hq, int Nq);
hipError_t launch_bwd_bf16(const BwdArgs& a, hipStream_t stream);

// Gradients of the packed-sequence forward (layouts of FwdVarlenArgs; the
// workspace is bwd_workspace_bytes(1, Hq, total_q)).
struct BwdVarlenArgs {
  const void* q;
  const void* k;
  const void* v;
  const void* out;
  const void* dout;
  const float* lse;
  void* dq;
  void* dk;
  void* dv;
  const int* cu_seqlens_q;
  const int* cu_seqlens_k;
  int n_seqs, total_q, total_k, Hq, Hkv, d;
  int causal, window;
  float scale;
  void* workspace;
};

hipError_t launch_bwd_bf16_varlen(const BwdVarlenArgs& a, hipStream_t stream);

size_t decode_workspace_bytes(int B, int Hq, int d, int block_size, int max_blocks_per_seq);
hipError_t launch_decode_paged(const DecodeArgs& a, hipStream_t stream);
// The same launch with the library's own per-device scratch array as the
// workspace (a.workspace is ignored); needs decode_workspace_bytes(...) <=
// decode_scratch_bytes(), which the caller checks.
size_t decode_scratch_bytes();
hipError_t launch_decode_paged_noalloc(const DecodeArgs& a, hipStream_t stream);

}  // namespace attn
