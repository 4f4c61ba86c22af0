// Verification index-set selection (Dustin page, methodology 1: hybrid
// attention aggregation; verification workflow step 3 forms the compressed
// cache from these positions).
//
// One workgroup (1024 threads) per (sequence b, KV head g).  Of the
// positions [0, c): the first n_sink and the last n_recent are kept; of the
// middle ones, the m best by the draft-lookahead score, then the best
// remaining ones by the target-historical score until n_sel are chosen.
// "Best": higher score, NaN below every number, -0 equal to +0, ties to the
// lower position.  The chosen positions are marked in an LDS bitmap and
// written out ascending; if fewer than n_sel exist the tail is -1.
//
// Each "k best" is an exact radix select: scores become order-preserving
// 32-bit keys; four passes of 8-bit digit histograms (per-wave LDS
// sub-histograms) find the key T of the k-th best candidate and how many
// candidates equal to T are still needed; one position-ordered pass then
// marks every candidate above T and the lowest-positioned ones equal to T
// (ranks from a block-wide scan of the equality flags).  Scores are read
// from global memory on every pass; after the first they come from L2.
#include "common.hpp"
#include "launch.h"

namespace hsv {
namespace {

constexpr int kSelThreads = 1024;
constexpr int kSelWaves = kSelThreads / kWave;

// Order-preserving key: larger score -> larger key; NaN -> 0 (below every
// number, -inf included); -0 -> the key of +0.
__device__ __forceinline__ uint32_t order_key(float f) {
  if (f != f) return 0u;
  uint32_t u = __float_as_uint(f == 0.f ? 0.f : f);
  return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}

// Exclusive prefix sum of `x` over the workgroup, in thread order; `total`
// receives the sum.  Uses `scratch` (kSelWaves words).
__device__ __forceinline__ uint32_t block_exclusive_scan(uint32_t x, uint32_t *scratch,
                                                         uint32_t *total) {
  const int lane = threadIdx.x % kWave, wave = threadIdx.x / kWave;
  uint32_t incl = x;
#pragma unroll
  for (int off = 1; off < kWave; off <<= 1) {
    const uint32_t y = __shfl_up(incl, off, kWave);
    if (lane >= off) incl += y;
  }
  if (lane == kWave - 1) scratch[wave] = incl;
  __syncthreads();
  uint32_t wave_base = 0, all = 0;
  for (int w = 0; w < kSelWaves; ++w) {
    const uint32_t s = scratch[w];
    if (w < wave) wave_base += s;
    all += s;
  }
  __syncthreads();
  *total = all;
  return wave_base + incl - x;
}

struct SelShared {
  uint32_t hist[kSelWaves][256];
  uint32_t tot[256];
  uint32_t scan[kSelWaves];
  uint32_t digit, need;
};

// Mark the k best candidates of rows[lo, hi) that are not yet in `bits`.
__device__ void select_best(const float *row, int lo, int hi, uint32_t k, uint32_t *bits,
                            SelShared &sh) {
  if (k == 0) return;
  const int tid = threadIdx.x, wave = tid / kWave;
  uint32_t prefix = 0, pmask = 0, need = k;
  for (int shift = 24; shift >= 0; shift -= 8) {
    for (int i = tid; i < kSelWaves * 256; i += kSelThreads) (&sh.hist[0][0])[i] = 0u;
    __syncthreads();
    for (int p = lo + tid; p < hi; p += kSelThreads) {
      if ((bits[p >> 5] >> (p & 31)) & 1u) continue;
      const uint32_t key = order_key(row[p]);
      if ((key & pmask) == prefix) atomicAdd(&sh.hist[wave][(key >> shift) & 255u], 1u);
    }
    __syncthreads();
    if (tid < 256) {
      uint32_t s = 0;
#pragma unroll
      for (int w = 0; w < kSelWaves; ++w) s += sh.hist[w][tid];
      sh.tot[tid] = s;
    }
    __syncthreads();
    if (tid == 0) {
      // digit d with (count above d) < need <= (count above d) + tot[d]
      uint32_t above = 0;
      int d = 255;
      for (; d > 0; --d) {
        if (above + sh.tot[d] >= need) break;
        above += sh.tot[d];
      }
      sh.digit = static_cast<uint32_t>(d);
      sh.need = need - above;
    }
    __syncthreads();
    prefix |= sh.digit << shift;
    pmask |= 255u << shift;
    need = sh.need;
    __syncthreads();
  }
  // prefix is the k-th best key; `need` candidates equal to it are taken,
  // lowest positions first
  uint32_t taken_eq = 0;
  for (int base = lo; base < hi; base += kSelThreads) {
    const int p = base + tid;
    bool gt = false, eq = false;
    if (p < hi && !((bits[p >> 5] >> (p & 31)) & 1u)) {
      const uint32_t key = order_key(row[p]);
      gt = key > prefix;
      eq = key == prefix;
    }
    uint32_t n_eq;
    const uint32_t rank = block_exclusive_scan(eq ? 1u : 0u, sh.scan, &n_eq);
    if (gt || (eq && taken_eq + rank < need)) atomicOr(&bits[p >> 5], 1u << (p & 31));
    taken_eq += n_eq;
    __syncthreads();
  }
  __syncthreads();
}

__global__ __launch_bounds__(kSelThreads) void select_kv_idx_kernel(
    const float *draft, const float *target, int score_len, const int32_t *ctx_lens, int hkv,
    int n_sel, int n_sink, int n_recent, int n_draft_top, int32_t *kv_idx) {
  extern __shared__ uint32_t bits[];  // ceil(score_len / 32) words
  __shared__ SelShared sh;
  const int tid = threadIdx.x;
  const int bg = blockIdx.x;
  const int b = bg / hkv;
  const int c = min(max(ctx_lens[b], 0), score_len);
  const int lo = min(n_sink, c);
  const int hi = max(c - n_recent, lo);
  const int n_protected = lo + (c - hi);
  const int fill = n_sel - n_protected;
  const int n_cand = hi - lo;
  const int m = min(min(n_draft_top, fill), n_cand);
  const int rest = min(fill - m, n_cand - m);

  const int words = (c + 31) / 32;
  for (int w = tid; w < words; w += kSelThreads) {
    // protected positions: [0, lo) and [hi, c)
    uint32_t v = 0;
    const int p0 = 32 * w;
#pragma unroll 4
    for (int j = 0; j < 32; ++j) {
      const int p = p0 + j;
      if (p < c && (p < lo || p >= hi)) v |= 1u << j;
    }
    bits[w] = v;
  }
  __syncthreads();

  const int64_t row0 = static_cast<int64_t>(bg) * score_len;
  select_best(draft + row0, lo, hi, static_cast<uint32_t>(m), bits, sh);
  select_best(target + row0, lo, hi, static_cast<uint32_t>(rest), bits, sh);

  // ascending compaction: thread t owns a contiguous run of words
  const int per = (words + kSelThreads - 1) / kSelThreads;
  const int w0 = min(tid * per, words), w1 = min(w0 + per, words);
  uint32_t cnt = 0;
  for (int w = w0; w < w1; ++w) cnt += __popc(bits[w]);
  uint32_t total;
  uint32_t out = block_exclusive_scan(cnt, sh.scan, &total);
  int32_t *dst = kv_idx + static_cast<int64_t>(bg) * n_sel;
  for (int w = w0; w < w1; ++w) {
    uint32_t v = bits[w];
    while (v) {
      const int j = __ffs(v) - 1;
      v &= v - 1;
      if (out < static_cast<uint32_t>(n_sel)) dst[out] = 32 * w + j;
      ++out;
    }
  }
  for (int s = static_cast<int>(total) + tid; s < n_sel; s += kSelThreads) dst[s] = -1;
}

}  // namespace

int select_max_positions() { return 1 << 19; }

hipError_t launch_select_kv_idx(const float *draft, const float *target, int score_len,
                                const int32_t *ctx_lens, int batch, int hkv, int n_sel,
                                int n_sink, int n_recent, int n_draft_top, int32_t *kv_idx,
                                hipStream_t s) {
  const size_t lds = static_cast<size_t>((score_len + 31) / 32) * sizeof(uint32_t);
  hipLaunchKernelGGL(select_kv_idx_kernel, dim3(static_cast<unsigned>(batch * hkv)),
                     dim3(kSelThreads), lds, s, draft, target, score_len, ctx_lens, hkv, n_sel,
                     n_sink, n_recent, n_draft_top, kv_idx);
  return hipGetLastError();
}

}  // namespace hsv
