// C ABI of the attention library: argument validation, then dispatch to the
// gfx950 kernels.  Validation runs entirely on the host before any HIP call.
#include "attn.h"

#include <atomic>
#include <climits>

#include "launch.h"
#include "merge.h"

namespace {

int check_common(int B, int Hq, int Hkv, int d) {
  if (B < 0 || Hq < 1 || Hkv < 1) return ATTN_E_SHAPE;
  if (Hq % Hkv != 0) return ATTN_E_SHAPE;
  if (d != 64 && d != 128) return ATTN_E_HEADDIM;
  return ATTN_OK;
}

int check_fwd(const void* q, const void* k, const void* v, const void* out, int B, int Hq,
              int Hkv, int Nq, int Nk, int d, int causal, int window, long long grid) {
  int st = check_common(B, Hq, Hkv, d);
  if (st != ATTN_OK) return st;
  if (Nq < 0 || Nk < 0) return ATTN_E_SHAPE;
  // pointers of empty tensors may be NULL
  if ((long long)B * Nq > 0 && (!q || !out)) return ATTN_E_NULL;
  if ((long long)B * Nk > 0 && (!k || !v)) return ATTN_E_NULL;
  if (causal != 0 && causal != 1) return ATTN_E_MASK;
  if (window > 0 && !causal) return ATTN_E_MASK;
  if (causal && Nq > Nk) return ATTN_E_SHAPE;
  if (grid > INT_MAX) return ATTN_E_SHAPE;
  // a 64-key tile of one head is addressed with 32-bit byte offsets
  if ((long long)Hkv * d > (1LL << 22)) return ATTN_E_SHAPE;
  return ATTN_OK;
}

int fwd_common(const void* q, const void* k, const void* v, void* out, float* lse, int B, int Hq,
               int Hkv, int Nq, int Nk, int d, int causal, int window, float scale, void* stream,
               bool f32) {
  const long long grid =
      (B >= 0 && Hq >= 1 && Nq >= 0)
          ? (f32 ? attn::fwd_f32_grid(B, Hq, Nq) : attn::fwd_bf16_grid(B, Hq, Nq))
          : 0;
  const int st = check_fwd(q, k, v, out, B, Hq, Hkv, Nq, Nk, d, causal, window, grid);
  if (st != ATTN_OK) return st;
  if (B == 0 || Nq == 0) return ATTN_OK;
  attn::FwdArgs a{q, k, v, out, lse, B, Hq, Hkv, Nq, Nk, d, causal, window > 0 ? window : 0,
                  scale};
  const hipError_t e = f32 ? attn::launch_fwd_f32(a, static_cast<hipStream_t>(stream))
                           : attn::launch_fwd_bf16(a, static_cast<hipStream_t>(stream));
  return e == hipSuccess ? ATTN_OK : ATTN_E_LAUNCH;
}

}  // namespace

namespace attn {

int device_cus() {
  // per-device CU count, looked up once (racing first calls store the same value)
  static std::atomic<int> cached[64];
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return 256;
  int cus = cached[dev].load(std::memory_order_relaxed);
  if (cus == 0) {
    if (hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess ||
        cus <= 0)
      cus = 256;
    cached[dev].store(cus, std::memory_order_relaxed);
  }
  return cus;
}

}  // namespace attn

extern "C" {

int attn_fwd(const void* q, const void* k, const void* v, void* out, float* lse, int B, int Hq,
             int Hkv, int Nq, int Nk, int d, int causal, int window, float scale, void* stream) {
  return fwd_common(q, k, v, out, lse, B, Hq, Hkv, Nq, Nk, d, causal, window, scale, stream,
                    false);
}

int attn_fwd_f32(const float* q, const float* k, const float* v, float* out, float* lse, int B,
                 int Hq, int Hkv, int Nq, int Nk, int d, int causal, int window, float scale,
                 void* stream) {
  return fwd_common(q, k, v, out, lse, B, Hq, Hkv, Nq, Nk, d, causal, window, scale, stream,
                    true);
}

int attn_fwd_varlen(const void* q, const void* k, const void* v, void* out, float* lse,
                    const int* cu_seqlens_q, const int* cu_seqlens_k, int num_seqs, int total_q,
                    int total_k, int Hq, int Hkv, int d, int causal, int window, float scale,
                    void* stream) {
  // the per-sequence lengths live on the device: the host checks the totals
  if (num_seqs < 0 || total_q < 0 || total_k < 0) return ATTN_E_SHAPE;
  const int st = check_common(num_seqs, Hq, Hkv, d);
  if (st != ATTN_OK) return st;
  if (causal != 0 && causal != 1) return ATTN_E_MASK;
  if (window > 0 && !causal) return ATTN_E_MASK;
  if (attn::fwd_bf16_varlen_grid(num_seqs, Hq, total_q) > INT_MAX) return ATTN_E_SHAPE;
  if ((long long)Hkv * d > (1LL << 22)) return ATTN_E_SHAPE;
  if (num_seqs == 0 || total_q == 0) return ATTN_OK;
  if (!q || !out || !cu_seqlens_q || !cu_seqlens_k) return ATTN_E_NULL;
  if (total_k > 0 && (!k || !v)) return ATTN_E_NULL;
  attn::FwdVarlenArgs a{q,        k,       v,       out, lse, cu_seqlens_q, cu_seqlens_k,
                        num_seqs, total_q, total_k, Hq,  Hkv, d,            causal,
                        window > 0 ? window : 0,    scale};
  const hipError_t e = attn::launch_fwd_bf16_varlen(a, static_cast<hipStream_t>(stream));
  return e == hipSuccess ? ATTN_OK : ATTN_E_LAUNCH;
}

size_t attn_prefill_paged_workspace_size(int num_seqs, int total_q, int Hq, int d, int block_size,
                                         int max_blocks_per_seq) {
  if (num_seqs < 0 || total_q < 0 || Hq < 1 || (d != 64 && d != 128) || block_size != 16 ||
      max_blocks_per_seq < 1 || (long long)max_blocks_per_seq * block_size > INT_MAX)
    return 0;
  return attn::prefill_paged_workspace_bytes(num_seqs, Hq, total_q, d, max_blocks_per_seq);
}

int attn_prefill_paged(const void* q, const void* kcache, const void* vcache,
                       const int* block_table, const int* seq_lens, const int* cu_seqlens_q,
                       void* out, float* lse, int num_seqs, int total_q, int Hq, int Hkv, int d,
                       int block_size, int max_blocks_per_seq, int num_blocks, int window,
                       float scale, void* workspace, size_t workspace_bytes, void* stream) {
  if (num_seqs < 0 || total_q < 0) return ATTN_E_SHAPE;
  const int st = check_common(num_seqs, Hq, Hkv, d);
  if (st != ATTN_OK) return st;
  if (block_size != 16 || max_blocks_per_seq < 1 || num_blocks < 1) return ATTN_E_SHAPE;
  if ((long long)max_blocks_per_seq * block_size > INT_MAX) return ATTN_E_SHAPE;
  if ((long long)num_seqs * max_blocks_per_seq > INT_MAX) return ATTN_E_SHAPE;
  if (attn::prefill_paged_grid(num_seqs, Hq, total_q, max_blocks_per_seq) > INT_MAX)
    return ATTN_E_SHAPE;
  if ((long long)Hkv * d > (1LL << 22)) return ATTN_E_SHAPE;
  if (num_seqs == 0 || total_q == 0) return ATTN_OK;
  if (!q || !out || !kcache || !vcache || !block_table || !seq_lens || !cu_seqlens_q)
    return ATTN_E_NULL;
  const size_t need =
      attn::prefill_paged_workspace_bytes(num_seqs, Hq, total_q, d, max_blocks_per_seq);
  if (need > 0 && (!workspace || workspace_bytes < need)) return ATTN_E_WORKSPACE;
  attn::PrefillPagedArgs a{q,           kcache,   vcache,          block_table, seq_lens,
                           cu_seqlens_q, out,     lse,             num_seqs,    total_q,
                           Hq,           Hkv,     d,               max_blocks_per_seq,
                           num_blocks,   window > 0 ? window : 0,  scale,       workspace};
  const hipError_t e = attn::launch_prefill_paged(a, static_cast<hipStream_t>(stream));
  return e == hipSuccess ? ATTN_OK : ATTN_E_LAUNCH;
}

int attn_bwd_varlen(const void* q, const void* k, const void* v, const void* out,
                    const void* dout, const float* lse, void* dq, void* dk, void* dv,
                    const int* cu_seqlens_q, const int* cu_seqlens_k, int num_seqs, int total_q,
                    int total_k, int Hq, int Hkv, int d, int causal, int window, float scale,
                    void* workspace, size_t workspace_bytes, void* stream) {
  if (num_seqs < 0 || total_q < 0 || total_k < 0) return ATTN_E_SHAPE;
  const int st = check_common(num_seqs, Hq, Hkv, d);
  if (st != ATTN_OK) return st;
  if (causal != 0 && causal != 1) return ATTN_E_MASK;
  if (window > 0 && !causal) return ATTN_E_MASK;
  if (Hq > 65535) return ATTN_E_SHAPE;  // grid y
  // schedule slots of both packed axes fit the grid's x dimension
  if ((long long)total_q / 128 + num_seqs > INT_MAX || (long long)total_k / 128 + num_seqs > INT_MAX)
    return ATTN_E_SHAPE;
  if ((long long)total_q * Hq * d > (1LL << 40) || (long long)Hkv * d > (1LL << 22))
    return ATTN_E_SHAPE;
  if (num_seqs == 0 || (total_q == 0 && total_k == 0)) return ATTN_OK;
  if (!cu_seqlens_q || !cu_seqlens_k) return ATTN_E_NULL;
  if (total_q > 0 && (!q || !out || !dout || !lse || !dq)) return ATTN_E_NULL;
  if (total_k > 0 && (!k || !v || !dk || !dv)) return ATTN_E_NULL;
  const size_t need = attn::bwd_workspace_bytes(1, Hq, total_q);
  if (need > 0 && (!workspace || workspace_bytes < need)) return ATTN_E_WORKSPACE;
  attn::BwdVarlenArgs a{q,        k,        v,          out,          dout,
                        lse,      dq,       dk,         dv,           cu_seqlens_q,
                        cu_seqlens_k, num_seqs, total_q, total_k,    Hq,
                        Hkv,      d,        causal,     window > 0 ? window : 0,
                        scale,    workspace};
  const hipError_t e = attn::launch_bwd_bf16_varlen(a, static_cast<hipStream_t>(stream));
  return e == hipSuccess ? ATTN_OK : ATTN_E_LAUNCH;
}

int attn_merge(const void* o_a, const float* lse_a, const void* o_b, const float* lse_b,
               void* out, float* lse_out, int B, int N, int H, int d, void* stream) {
  if (B < 0 || N < 0 || H < 1) return ATTN_E_SHAPE;
  if (d != 64 && d != 128) return ATTN_E_HEADDIM;
  if ((long long)B * N * H * d > (1LL << 40)) return ATTN_E_SHAPE;
  if ((long long)B * N == 0) return ATTN_OK;
  if (!o_a || !lse_a || !o_b || !lse_b || !out) return ATTN_E_NULL;
  attn::MergeArgs a{o_a, lse_a, o_b, lse_b, out, lse_out, B, N, H, d};
  const hipError_t e = attn::launch_merge(a, static_cast<hipStream_t>(stream));
  return e == hipSuccess ? ATTN_OK : ATTN_E_LAUNCH;
}

size_t attn_decode_paged_workspace_size(int B, int Hq, int d, int block_size,
                                        int max_blocks_per_seq) {
  if (B < 0 || Hq < 1 || (d != 64 && d != 128) || block_size != 16 || max_blocks_per_seq < 1)
    return 0;
  if ((long long)max_blocks_per_seq * block_size > INT_MAX) return 0;
  return attn::decode_workspace_bytes(B, Hq, d, block_size, max_blocks_per_seq);
}

}  // extern "C"

namespace {

int check_decode(const void* q, const void* kcache, const void* vcache, const int* block_table,
                 const int* seq_lens, const void* out, int B, int Hq, int Hkv, int d,
                 int block_size, int max_blocks_per_seq, int num_blocks) {
  int st = check_common(B, Hq, Hkv, d);
  if (st != ATTN_OK) return st;
  if (B > 0 && (!q || !kcache || !vcache || !block_table || !seq_lens || !out))
    return ATTN_E_NULL;
  if (block_size != 16 || max_blocks_per_seq < 1 || num_blocks < 1) return ATTN_E_SHAPE;
  if ((long long)max_blocks_per_seq * block_size > INT_MAX) return ATTN_E_SHAPE;
  if (B > 65535 || Hq > 65535) return ATTN_E_SHAPE;  // grid y limits
  // block counts of the whole batch are summed in 32-bit integers on the device
  if ((long long)B * max_blocks_per_seq > INT_MAX) return ATTN_E_SHAPE;
  return ATTN_OK;
}

}  // namespace

extern "C" {

int attn_decode_paged(const void* q, const void* kcache, const void* vcache,
                      const int* block_table, const int* seq_lens, void* out, float* lse, int B,
                      int Hq, int Hkv, int d, int block_size, int max_blocks_per_seq,
                      int num_blocks, int window, float scale, void* workspace,
                      size_t workspace_bytes, void* stream) {
  const int st = check_decode(q, kcache, vcache, block_table, seq_lens, out, B, Hq, Hkv, d,
                              block_size, max_blocks_per_seq, num_blocks);
  if (st != ATTN_OK) return st;
  if (B == 0) return ATTN_OK;
  const size_t need = attn::decode_workspace_bytes(B, Hq, d, block_size, max_blocks_per_seq);
  if (!workspace || workspace_bytes < need) return ATTN_E_WORKSPACE;
  attn::DecodeArgs a{q,  kcache, vcache, block_table, seq_lens, out, lse,
                     B,  Hq,     Hkv,    d,           block_size, max_blocks_per_seq,
                     num_blocks, window > 0 ? window : 0, scale, workspace};
  const hipError_t e = attn::launch_decode_paged(a, static_cast<hipStream_t>(stream));
  return e == hipSuccess ? ATTN_OK : ATTN_E_LAUNCH;
}

int attn_decode_paged_noalloc(const void* q, const void* kcache, const void* vcache,
                              const int* block_table, const int* seq_lens, void* out, float* lse,
                              int B, int Hq, int Hkv, int d, int block_size,
                              int max_blocks_per_seq, int num_blocks, int window, float scale,
                              void* stream) {
  const int st = check_decode(q, kcache, vcache, block_table, seq_lens, out, B, Hq, Hkv, d,
                              block_size, max_blocks_per_seq, num_blocks);
  if (st != ATTN_OK) return st;
  if (B == 0) return ATTN_OK;
  if (attn::decode_workspace_bytes(B, Hq, d, block_size, max_blocks_per_seq) >
      attn::decode_scratch_bytes())
    return ATTN_E_WORKSPACE;
  attn::DecodeArgs a{q,  kcache, vcache, block_table, seq_lens, out, lse,
                     B,  Hq,     Hkv,    d,           block_size, max_blocks_per_seq,
                     num_blocks, window > 0 ? window : 0, scale, nullptr};
  const hipError_t e = attn::launch_decode_paged_noalloc(a, static_cast<hipStream_t>(stream));
  return e == hipSuccess ? ATTN_OK : ATTN_E_LAUNCH;
}

size_t attn_bwd_workspace_size(int B, int Hq, int Nq) {
  if (B < 0 || Hq < 1 || Nq < 0) return 0;
  return attn::bwd_workspace_bytes(B, Hq, Nq);
}

int attn_bwd(const void* q, const void* k, const void* v, const void* out, const void* dout,
             const float* lse, void* dq, void* dk, void* dv, int B, int Hq, int Hkv, int Nq,
             int Nk, int d, int causal, int window, float scale, void* workspace,
             size_t workspace_bytes, void* stream) {
  const int st = check_fwd(q, k, v, dq, B, Hq, Hkv, Nq, Nk, d, causal, window, 0);
  if (st != ATTN_OK) return st;
  if ((long long)B * Nq > 0 && (!out || !dout || !lse)) return ATTN_E_NULL;
  if ((long long)B * Nk > 0 && (!dk || !dv)) return ATTN_E_NULL;
  if (B > 65535 || Hq > 65535 || Hkv > 65535) return ATTN_E_SHAPE;  // grid y, z limits
  if ((long long)B * Nq * Hq * d > (1LL << 40)) return ATTN_E_SHAPE;
  if (B == 0 || (Nq == 0 && Nk == 0)) return ATTN_OK;
  const size_t need = attn::bwd_workspace_bytes(B, Hq, Nq);
  if (need > 0 && (!workspace || workspace_bytes < need)) return ATTN_E_WORKSPACE;
  attn::BwdArgs a{q, k, v, out, dout, lse, dq, dk, dv, B, Hq, Hkv, Nq, Nk, d,
                  causal, window > 0 ? window : 0, scale, workspace};
  const hipError_t e = attn::launch_bwd_bf16(a, static_cast<hipStream_t>(stream));
  return e == hipSuccess ? ATTN_OK : ATTN_E_LAUNCH;
}

int attn_set_fwd_sched_slots(int n) { return attn::set_fwd_sched_slots(n); }

const char* attn_status_str(int status) {
  switch (status) {
    case ATTN_OK: return "ok";
    case ATTN_E_NULL: return "a required pointer is NULL";
    case ATTN_E_SHAPE: return "invalid or unsupported sizes";
    case ATTN_E_HEADDIM: return "head dimension must be 64 or 128";
    case ATTN_E_MASK: return "invalid mask (window requires causal; causal is 0 or 1)";
    case ATTN_E_WORKSPACE: return "workspace missing or too small";
    case ATTN_E_LAUNCH: return "HIP launch failed";
    default: return "unknown status";
  }
}

}  // extern "C"
