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
// The move is in place.  Parents precede children, so p_t >= t: writing row
// c_b + t can only clobber the source of an earlier entry s < t (when
// p_s = t), never a later one (p_s >= s > t).  Each workgroup therefore moves
// its (sequence, KV head)'s path in chunks of increasing t: every source row
// of a chunk is staged in LDS, then, after a barrier, every destination row
// of the chunk is written.  The leading entries with p_t == t (the path
// begins 0, 1, ...) are already in place and skipped.  The context lengths
// are bumped by a second launch, after every workgroup has read them.
//
// Trees of up to 256 nodes: parents are read into LDS and each path or
// depth is found by walking parent pointers (a valid array strictly
// decreases along them).
#include "common.hpp"
#include "launch.h"

namespace hsv {
namespace {

constexpr int kMaxNodes = 256;
constexpr int kAcceptThreads = 256;
constexpr int kAcceptMaxRowWords = 128;               // 512-byte rows: D 128, fp32
constexpr int kStageWords = 64 * kAcceptMaxRowWords;  // 32 KB: 64 to 256 rows per chunk

// Parents of sequence b into par[0, n), and whether any is out of range
// ([-1, i-1]).  Called by a whole workgroup; ends with a barrier.
__device__ __forceinline__ bool load_parents(const int32_t *parent_row, int n, int32_t *par,
                                             int32_t *bad_sh) {
  const int tid = threadIdx.x;
  if (tid == 0) *bad_sh = 0;
  __syncthreads();
  for (int i = tid; i < n; i += blockDim.x) {
    const int p = parent_row[i];
    par[i] = p;
    if (p < -1 || p >= i) atomicOr(bad_sh, 1);
  }
  __syncthreads();
  return *bad_sh != 0;
}

// Depth of node i (the node itself counts; a child of the prefix has 1).
__device__ __forceinline__ int node_depth(const int32_t *par, int i) {
  int d = 0;
  for (int j = i; j >= 0; j = par[j]) ++d;
  return d;
}

// Position ids: one 256-thread workgroup per sequence, thread i for node i;
// every entry of a sequence with an invalid parent array is -1.
__global__ __launch_bounds__(kMaxNodes) void tree_position_kernel(const int32_t *parent,
                                                                  const int32_t *ctx_lens,
                                                                  int32_t *pos, int n) {
  __shared__ int32_t par[kMaxNodes];
  __shared__ int32_t bad;
  const int b = blockIdx.x, i = threadIdx.x;
  const bool invalid = load_parents(parent + static_cast<int64_t>(b) * n, n, par, &bad);
  if (i < n)
    pos[static_cast<int64_t>(b) * n + i] = invalid ? -1 : ctx_lens[b] + node_depth(par, i) - 1;
}

// The accepted path of sequence b into path[0, len) (root side first), or
// len = 0 when the sequence is left unchanged (nothing accepted, a node out
// of range, an invalid parent array, or draft rows that would not fit the
// cache).  Called by a whole workgroup; ends with a barrier.
__device__ __forceinline__ int accepted_path(const int32_t *parent_row, int n, int a, int c,
                                             int s_cap, int32_t *par, int32_t *path,
                                             int32_t *bad_sh, int32_t *len_sh) {
  const bool invalid = load_parents(parent_row, n, par, bad_sh);
  if (threadIdx.x == 0) {
    int len = 0;
    if (!invalid && a >= 0 && a < n && c >= 0 && c <= s_cap - n) {
      len = node_depth(par, a);
      int t = len;
      for (int j = a; j >= 0; j = par[j]) path[--t] = j;
    }
    *len_sh = len;
  }
  __syncthreads();
  return *len_sh;
}

__global__ __launch_bounds__(kAcceptThreads) void accept_copy_kernel(
    uint32_t *k, uint32_t *v, const int32_t *ctx_lens, const int32_t *parent,
    const int32_t *accept_node, int hkv, int s_cap, int row_words, int n) {
  __shared__ uint32_t stage[kStageWords];
  __shared__ int32_t par[kMaxNodes], path[kMaxNodes];
  __shared__ int32_t bad, len_sh;
  const int bg = blockIdx.x, b = bg / hkv;
  const int tid = threadIdx.x;
  const int c = ctx_lens[b];
  const int len = accepted_path(parent + static_cast<int64_t>(b) * n, n, accept_node[b], c,
                                s_cap, par, path, &bad, &len_sh);
  int skip = 0;  // the path starts 0, 1, ..., skip - 1: those rows are in place
  while (skip < len && path[skip] == skip) ++skip;
  const int chunk = kStageWords / row_words;  // path entries per chunk
  for (int half = 0; half < 2; ++half) {
    uint32_t *rows = (half == 0 ? k : v) + (static_cast<int64_t>(bg) * s_cap + c) * row_words;
    for (int t0 = skip; t0 < len; t0 += chunk) {
      const int total = (min(len, t0 + chunk) - t0) * row_words;
      for (int i = tid; i < total; i += kAcceptThreads) {
        const int t = t0 + i / row_words, w = i % row_words;
        stage[i] = rows[static_cast<int64_t>(path[t]) * row_words + w];
      }
      __syncthreads();
      for (int i = tid; i < total; i += kAcceptThreads) {
        const int t = t0 + i / row_words, w = i % row_words;
        rows[static_cast<int64_t>(t) * row_words + w] = stage[i];
      }
      __syncthreads();
    }
  }
}

__global__ __launch_bounds__(kAcceptThreads) void accept_bump_kernel(int32_t *ctx_lens,
                                                                     const int32_t *parent,
                                                                     const int32_t *accept_node,
                                                                     int n, int s_cap) {
  __shared__ int32_t par[kMaxNodes], path[kMaxNodes];
  __shared__ int32_t bad, len_sh;
  const int b = blockIdx.x;
  const int c = ctx_lens[b];
  const int len = accepted_path(parent + static_cast<int64_t>(b) * n, n, accept_node[b], c,
                                s_cap, par, path, &bad, &len_sh);
  if (threadIdx.x == 0) ctx_lens[b] = c + len;
}

}  // namespace

hipError_t launch_tree_position_ids(const int32_t *parent, const int32_t *ctx_lens,
                                    int32_t *pos_ids, int batch, int n_draft, hipStream_t s) {
  if (n_draft < 1 || n_draft > kMaxNodes) return hipErrorInvalidValue;
  hipLaunchKernelGGL(tree_position_kernel, dim3(static_cast<unsigned>(batch)), dim3(kMaxNodes), 0,
                     s, parent, ctx_lens, pos_ids, n_draft);
  return hipGetLastError();
}

hipError_t launch_accept_path(void *k_cache, void *v_cache, int32_t *ctx_lens,
                              const int32_t *parent, const int32_t *accept_node, int batch,
                              int hkv, int s_cap, int row_bytes, int n_draft, hipStream_t s) {
  if (row_bytes % 4 != 0 || row_bytes / 4 > kAcceptMaxRowWords) return hipErrorInvalidValue;
  if (n_draft < 1 || n_draft > kMaxNodes) return hipErrorInvalidValue;
  hipLaunchKernelGGL(accept_copy_kernel, dim3(static_cast<unsigned>(batch * hkv)),
                     dim3(kAcceptThreads), 0, s, static_cast<uint32_t *>(k_cache),
                     static_cast<uint32_t *>(v_cache), ctx_lens, parent, accept_node, hkv, s_cap,
                     row_bytes / 4, n_draft);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(accept_bump_kernel, dim3(static_cast<unsigned>(batch)),
                     dim3(kAcceptThreads), 0, s, ctx_lens, parent, accept_node, n_draft, s_cap);
  return hipGetLastError();
}

}  // namespace hsv
