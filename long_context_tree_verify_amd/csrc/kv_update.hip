// Cache bookkeeping around a verification step.
//
// Position ids: a draft node takes position c_b + depth - 1, the place it
// would have in the sequence if its branch were accepted (LongSpec section
// 2.C: the draft tokens form a tree rooted at the cached prefix).
//
// Accepted-path update: the accepted tokens join the cache and the rejected
// ones are dropped (HiSpec page, reuse of the KV cache and hidden states;
// Dustin page, verification workflow step 5).  The draft rows sit at
// [c_b, c_b + N); the path p_0 < ... < p_{L-1} = a of the accepted node a
// (root side first) is moved so that row c_b + t receives row c_b + p_t, and
// c_b grows by L.  Rows at c_b + L and beyond are not written.
//
// The move is in place.  Since p_t >= t, a destination row can be the
// source of a later path entry, so each workgroup first stages every source
// row of its (sequence, KV head) in LDS, meets at a barrier, then writes.
// The leading entries with p_t == t (the path begins 0, 1, ...) are already
// in place and skipped.  The context lengths are bumped by a second launch,
// after every workgroup has read them.
#include "common.hpp"
#include "launch.h"

namespace hsv {
namespace {

constexpr int kAcceptThreads = 256;
constexpr int kAcceptMaxRowWords = 128;               // 512-byte rows: D 128, fp32
constexpr int kAcceptMaxWords = 64 * kAcceptMaxRowWords;

// One wave per sequence: pos = c_b + popcount(ancestor-or-self mask) - 1;
// every entry of a sequence with an invalid parent array is -1.
__global__ __launch_bounds__(64) void tree_position_kernel(const int32_t *parent,
                                                           const int32_t *ctx_lens, int32_t *pos,
                                                           int n) {
  const int b = blockIdx.x, lane = threadIdx.x;
  bool bad;
  const uint64_t anc = tree_ancestors(parent + static_cast<int64_t>(b) * n, n, lane, &bad);
  if (lane < n)
    pos[static_cast<int64_t>(b) * n + lane] = bad ? -1 : ctx_lens[b] + __popcll(anc) - 1;
}

// Bit j set iff draft node j is on the accepted path; 0 when the sequence is
// left unchanged (nothing accepted, node out of range, invalid parent array,
// or the draft rows would not fit the cache).  Called by a whole wave.
__device__ __forceinline__ uint64_t accepted_mask(const int32_t *parent_row, int n, int a, int c,
                                                  int s_cap, int lane) {
  bool bad;
  const uint64_t anc = tree_ancestors(parent_row, n, lane, &bad);
  if (bad || a < 0 || a >= n || c < 0 || c > s_cap - n) return 0;
  return shfl_u64(anc, a);
}

__global__ __launch_bounds__(kAcceptThreads) void accept_copy_kernel(
    uint32_t *k, uint32_t *v, const int32_t *ctx_lens, const int32_t *parent,
    const int32_t *accept_node, int hkv, int s_cap, int row_words, int n) {
  __shared__ uint32_t stage[kAcceptMaxWords];
  __shared__ int32_t path[64];
  __shared__ uint64_t mask_sh;
  const int bg = blockIdx.x, b = bg / hkv;
  const int tid = threadIdx.x;
  const int c = ctx_lens[b];
  if (tid < kWave) {
    const uint64_t m = accepted_mask(parent + static_cast<int64_t>(b) * n, n, accept_node[b], c,
                                     s_cap, tid);
    if ((m >> tid) & 1u) path[__popcll(m & ((uint64_t{1} << tid) - 1))] = tid;
    if (tid == 0) mask_sh = m;
  }
  __syncthreads();
  const uint64_t m = mask_sh;
  const int len = __popcll(m);
  const int skip = ~m == 0 ? 64 : __builtin_ctzll(~m);  // path starts 0, 1, ..., skip-1
  const int total = (len - skip) * row_words;
  if (total <= 0) return;
  for (int half = 0; half < 2; ++half) {
    uint32_t *rows = (half == 0 ? k : v) + (static_cast<int64_t>(bg) * s_cap + c) * row_words;
    for (int i = tid; i < total; i += kAcceptThreads) {
      const int t = skip + i / row_words, w = i % row_words;
      stage[i] = rows[static_cast<int64_t>(path[t]) * row_words + w];
    }
    __syncthreads();
    for (int i = tid; i < total; i += kAcceptThreads) {
      const int t = skip + i / row_words, w = i % row_words;
      rows[static_cast<int64_t>(t) * row_words + w] = stage[i];
    }
    __syncthreads();
  }
}

__global__ __launch_bounds__(64) void accept_bump_kernel(int32_t *ctx_lens, const int32_t *parent,
                                                         const int32_t *accept_node, int n,
                                                         int s_cap) {
  const int b = blockIdx.x, lane = threadIdx.x;
  const int c = ctx_lens[b];
  const uint64_t m = accepted_mask(parent + static_cast<int64_t>(b) * n, n, accept_node[b], c,
                                   s_cap, lane);
  if (lane == 0) ctx_lens[b] = c + __popcll(m);
}

}  // namespace

hipError_t launch_tree_position_ids(const int32_t *parent, const int32_t *ctx_lens,
                                    int32_t *pos_ids, int batch, int n_draft, hipStream_t s) {
  hipLaunchKernelGGL(tree_position_kernel, dim3(static_cast<unsigned>(batch)), dim3(kWave), 0, s,
                     parent, ctx_lens, pos_ids, n_draft);
  return hipGetLastError();
}

hipError_t launch_accept_path(void *k_cache, void *v_cache, int32_t *ctx_lens,
                              const int32_t *parent, const int32_t *accept_node, int batch,
                              int hkv, int s_cap, int row_bytes, int n_draft, hipStream_t s) {
  if (row_bytes % 4 != 0 || row_bytes / 4 > kAcceptMaxRowWords) return hipErrorInvalidValue;
  hipLaunchKernelGGL(accept_copy_kernel, dim3(static_cast<unsigned>(batch * hkv)),
                     dim3(kAcceptThreads), 0, s, static_cast<uint32_t *>(k_cache),
                     static_cast<uint32_t *>(v_cache), ctx_lens, parent, accept_node, hkv, s_cap,
                     row_bytes / 4, n_draft);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(accept_bump_kernel, dim3(static_cast<unsigned>(batch)), dim3(kWave), 0, s,
                     ctx_lens, parent, accept_node, n_draft, s_cap);
  return hipGetLastError();
}

}  // namespace hsv
