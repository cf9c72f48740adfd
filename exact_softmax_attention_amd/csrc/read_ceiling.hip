// Read-bandwidth ceiling of the paged decode's access pattern on this GPU.
//
// A measurement program, not part of the library: it reads the decode
// workload's bytes (37184 blocks of 32 KiB = 1.2185 GB, the K and V cache
// blocks the 16-sequence batch touches) out of a 40000-block pool and
// reports the best of 10 timed passes (HIP events) for three patterns:
//   contiguous   blocks 0 .. n-1 in order, each work group reading whole blocks
//   random       the same number of blocks through a random permutation of the
//                pool (the order a paged cache hands out blocks), whole blocks
//   per-head     random blocks again, but as the decode kernel reads them: a
//                block is 16 token rows of 8 heads x 256 bytes, and wave h of
//                a work group reads only head h's 256 bytes of each row (a
//                2 KiB stride), the 8 waves of a work group streaming their
//                slices of the same blocks without synchronising
// Each lane loads 16 bytes at a time with DEPTH blocks in flight per wave; the
// data is folded into one word per lane so that no load is dead.  Every
// pattern is measured with ordinary loads and with non-temporal loads (which
// the decode kernel uses: the cache is streamed once per call).
//
// Build: hipcc --offload-arch=gfx950 -O3 -o read_ceiling read_ceiling.hip
// Run:   ./read_ceiling      (one JSON line on stdout)
#include <hip/hip_runtime.h>

#include <algorithm>
#include <cstdio>
#include <random>
#include <vector>

namespace {

typedef unsigned u32x4 __attribute__((ext_vector_type(4)));
constexpr int kBlockBytes = 32768;
constexpr int kBlockVec = kBlockBytes / 16;  // 16-byte pieces per block
constexpr int kPoolBlocks = 40000;
constexpr int kReadBlocks = 37184;           // 1.2185 GB
constexpr int kThreads = 512;                // 8 waves

// whole blocks: a work group reads one block per step (each lane 4 pieces)
template <bool NT>
__device__ __forceinline__ u32x4 ld(const u32x4* p) {
  if constexpr (NT) return __builtin_nontemporal_load(p);
  else return *p;
}

template <int DEPTH, bool NT>
__global__ __launch_bounds__(kThreads) void read_whole(const u32x4* __restrict__ pool,
                                                       const int* __restrict__ ids, int n,
                                                       unsigned* __restrict__ sink) {
  const int tid = threadIdx.x;
  u32x4 acc = {0u, 0u, 0u, 0u};
  for (int b = blockIdx.x; b < n; b += gridDim.x * DEPTH) {
    u32x4 r[DEPTH][kBlockVec / kThreads];
#pragma unroll
    for (int d = 0; d < DEPTH; ++d) {
      const int bb = min(b + d * (int)gridDim.x, n - 1);
      const u32x4* p = pool + (size_t)ids[bb] * kBlockVec + tid;
#pragma unroll
      for (int j = 0; j < kBlockVec / kThreads; ++j) r[d][j] = ld<NT>(p + j * kThreads);
    }
#pragma unroll
    for (int d = 0; d < DEPTH; ++d)
#pragma unroll
      for (int j = 0; j < kBlockVec / kThreads; ++j) acc ^= r[d][j];
  }
  sink[blockIdx.x * kThreads + tid] = acc[0] ^ acc[1] ^ acc[2] ^ acc[3];
}

// per-head slices: wave h reads bytes [256 h, 256 h + 256) of each of the
// block's 16 rows of 2 KiB (lane: row lane / 16 + 4 i, piece lane % 16)
template <int DEPTH, bool NT>
__global__ __launch_bounds__(kThreads) void read_heads(const u32x4* __restrict__ pool,
                                                       const int* __restrict__ ids, int n,
                                                       unsigned* __restrict__ sink) {
  const int lane = threadIdx.x & 63, h = threadIdx.x >> 6;
  const int off = (lane >> 4) * 128 + h * 16 + (lane & 15);  // in 16-byte pieces
  u32x4 acc = {0u, 0u, 0u, 0u};
  for (int b = blockIdx.x; b < n; b += gridDim.x * DEPTH) {
    u32x4 r[DEPTH][4];
#pragma unroll
    for (int d = 0; d < DEPTH; ++d) {
      const int bb = min(b + d * (int)gridDim.x, n - 1);
      const u32x4* p = pool + (size_t)ids[bb] * kBlockVec + off;
#pragma unroll
      for (int i = 0; i < 4; ++i) r[d][i] = ld<NT>(p + i * 4 * 128);  // rows 4 i .. 4 i + 3
    }
#pragma unroll
    for (int d = 0; d < DEPTH; ++d)
#pragma unroll
      for (int i = 0; i < 4; ++i) acc ^= r[d][i];
  }
  sink[blockIdx.x * kThreads + threadIdx.x] = acc[0] ^ acc[1] ^ acc[2] ^ acc[3];
}

#define CHECK(x)                                                            \
  do {                                                                      \
    hipError_t e_ = (x);                                                    \
    if (e_ != hipSuccess) {                                                 \
      std::fprintf(stderr, "%s: %s\n", #x, hipGetErrorString(e_));          \
      std::exit(1);                                                         \
    }                                                                       \
  } while (0)

}  // namespace

int main() {
  u32x4* pool = nullptr;
  int* ids = nullptr;
  unsigned* sink = nullptr;
  int cus = 0;
  CHECK(hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, 0));
  const int max_grid = 4 * cus;
  CHECK(hipMalloc(&pool, (size_t)kPoolBlocks * kBlockBytes));
  CHECK(hipMalloc(&ids, kReadBlocks * sizeof(int)));
  CHECK(hipMalloc(&sink, (size_t)max_grid * kThreads * sizeof(unsigned)));
  CHECK(hipMemset(pool, 1, (size_t)kPoolBlocks * kBlockBytes));
  std::vector<int> seq(kReadBlocks), perm(kPoolBlocks);
  for (int i = 0; i < kReadBlocks; ++i) seq[i] = i;
  for (int i = 0; i < kPoolBlocks; ++i) perm[i] = i;
  std::mt19937 gen(5);
  std::shuffle(perm.begin(), perm.end(), gen);
  perm.resize(kReadBlocks);
  hipEvent_t e0, e1;
  CHECK(hipEventCreate(&e0));
  CHECK(hipEventCreate(&e1));

  // best GB/s over the grid sizes and 10 timed passes each
  auto best_of = [&](auto kernel, const std::vector<int>& order) {
    CHECK(hipMemcpy(ids, order.data(), kReadBlocks * sizeof(int), hipMemcpyHostToDevice));
    double best = 0;
    for (int grid : {cus, 2 * cus, max_grid}) {
      hipLaunchKernelGGL(kernel, dim3(grid), dim3(kThreads), 0, 0, pool, ids, kReadBlocks, sink);
      CHECK(hipGetLastError());
      CHECK(hipDeviceSynchronize());
      for (int it = 0; it < 10; ++it) {
        CHECK(hipEventRecord(e0, 0));
        hipLaunchKernelGGL(kernel, dim3(grid), dim3(kThreads), 0, 0, pool, ids, kReadBlocks, sink);
        CHECK(hipEventRecord(e1, 0));
        CHECK(hipEventSynchronize(e1));
        float ms = 0;
        CHECK(hipEventElapsedTime(&ms, e0, e1));
        best = std::max(best, (double)kReadBlocks * kBlockBytes / (ms * 1e-3) / 1e9);
      }
    }
    return best;
  };
  const double contiguous = std::max(best_of(read_whole<2, false>, seq), best_of(read_whole<4, false>, seq));
  const double random = std::max(best_of(read_whole<2, false>, perm), best_of(read_whole<4, false>, perm));
  const double heads = std::max(best_of(read_heads<2, false>, perm), best_of(read_heads<4, false>, perm));
  const double contiguous_nt = std::max(best_of(read_whole<2, true>, seq), best_of(read_whole<4, true>, seq));
  const double random_nt = std::max(best_of(read_whole<2, true>, perm), best_of(read_whole<4, true>, perm));
  const double heads_nt = std::max(best_of(read_heads<2, true>, perm), best_of(read_heads<4, true>, perm));
  std::printf("{\"bytes\": %lld, \"contiguous_GBps\": %.1f, \"random_blocks_GBps\": %.1f, "
              "\"per_head_slices_GBps\": %.1f, \"contiguous_nt_GBps\": %.1f, "
              "\"random_blocks_nt_GBps\": %.1f, \"per_head_slices_nt_GBps\": %.1f}\n",
              (long long)kReadBlocks * kBlockBytes, contiguous, random, heads, contiguous_nt,
              random_nt, heads_nt);
  CHECK(hipFree(pool));
  CHECK(hipFree(ids));
  CHECK(hipFree(sink));
  return 0;
}
