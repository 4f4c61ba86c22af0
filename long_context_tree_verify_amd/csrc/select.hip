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
// Each "k best" is an exact radix select over order-preserving 32-bit keys:
// digit histograms find the key T of the k-th best candidate and how many
// candidates equal to T are still needed; every candidate above T and the
// lowest-positioned ones equal to T are marked.
//
// Rows of up to 65536 positions (select_kv_idx_reg): each thread holds its
// positions' keys in registers (position j * 1024 + thread, j < KPT), so a
// score row is read from memory once.  Three passes of 11/11/10-bit digits
// count into eight interleaved LDS histogram copies (lane & 7 picks the
// copy, so at most eight lanes of one atomic instruction meet in a bin);
// ties at T are ranked by position from per-column ballots.
// Longer rows (select_kv_idx_stream): four 8-bit passes re-read the row
// from memory (L2 after the first) and ties are ranked chunk by chunk.
#include "common.hpp"
#include "launch.h"

namespace hsv {
namespace {

constexpr int kSelThreads = 1024;
constexpr int kSelWaves = kSelThreads / kWave;

// Order-preserving key: larger score -> larger key; NaN -> 1 (below every
// number, -inf included); -0 -> the key of +0.  No score maps to 0, which
// the register-resident form uses for "not a candidate".
__device__ __forceinline__ uint32_t order_key(float f) {
  if (f != f) return 1u;
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

// Streaming form: mark the k best candidates of rows[lo, hi) that are not
// yet in `bits`.
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

__global__ __launch_bounds__(kSelThreads) void select_kv_idx_stream(
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


// ---------------------------------------------------------------------------
// Register-resident form
// ---------------------------------------------------------------------------

constexpr int kBins = 2048;   // 11-bit digits
constexpr int kCopies = 8;    // histogram copies, interleaved: word = bin * 8 + copy

template <int KPT>
struct RegShared {
  uint32_t hist[kBins * kCopies];
  uint32_t colcnt[kSelWaves][64];   // per wave, per column: keys equal to T
  uint64_t bitmap[KPT * kSelWaves]; // entry e covers positions [64 e, 64 e + 64)
  uint32_t scan[kSelWaves];
  uint32_t digit, need, tot_eq, col_j, col_rem;
};

// The k-th largest (k >= 1) of this workgroup's keys that are >= floor
// (floor >= 1; at least k such keys must exist): three histogram passes of
// 11/11/10-bit digits.  need_out = how many keys equal to it are among the
// k largest; tot_eq_out = how many keys >= floor equal it.
template <int N, int KPT>
__device__ __forceinline__ uint32_t radix_kth(const uint32_t (&key)[N], uint32_t floor, uint32_t k,
                                              RegShared<KPT> &sh, uint32_t &need_out,
                                              uint32_t &tot_eq_out) {
  const int tid = threadIdx.x, lane = tid % kWave;
  const uint32_t copy = static_cast<uint32_t>(lane) & (kCopies - 1);
  uint32_t prefix = 0, pmask = 0, need = k, tot_eq = 0;
#pragma unroll
  for (int pass = 0; pass < 3; ++pass) {
    const int shift = pass == 0 ? 21 : (pass == 1 ? 10 : 0);
    const uint32_t dmask = pass == 2 ? 1023u : 2047u;
    uint4 *h4 = reinterpret_cast<uint4 *>(sh.hist);
    for (int i = tid; i < kBins * kCopies / 4; i += kSelThreads) h4[i] = make_uint4(0, 0, 0, 0);
    __syncthreads();
#pragma unroll
    for (int j = 0; j < N; ++j) {
      if (key[j] >= floor && (key[j] & pmask) == prefix)
        atomicAdd(&sh.hist[((key[j] >> shift) & dmask) * kCopies + copy], 1u);
    }
    __syncthreads();
    // thread t owns bins 2047 - 2t and 2046 - 2t: thread order is descending
    // bin order, so the exclusive scan counts the keys above a bin
    const int b_hi = kBins - 1 - 2 * tid, b_lo = b_hi - 1;
    const uint4 *hh = reinterpret_cast<const uint4 *>(sh.hist + b_hi * kCopies);
    const uint4 *hl = reinterpret_cast<const uint4 *>(sh.hist + b_lo * kCopies);
    const uint4 x0 = hh[0], x1 = hh[1], y0 = hl[0], y1 = hl[1];
    const uint32_t c_hi = x0.x + x0.y + x0.z + x0.w + x1.x + x1.y + x1.z + x1.w;
    const uint32_t c_lo = y0.x + y0.y + y0.z + y0.w + y1.x + y1.y + y1.z + y1.w;
    uint32_t total;
    const uint32_t above = block_exclusive_scan(c_hi + c_lo, sh.scan, &total);
    if (above < need && need <= above + c_hi) {
      sh.digit = static_cast<uint32_t>(b_hi);
      sh.need = need - above;
      sh.tot_eq = c_hi;
    } else if (above + c_hi < need && need <= above + c_hi + c_lo) {
      sh.digit = static_cast<uint32_t>(b_lo);
      sh.need = need - above - c_hi;
      sh.tot_eq = c_lo;
    }
    __syncthreads();
    prefix |= sh.digit << shift;
    pmask |= dmask << shift;
    need = sh.need;
    tot_eq = sh.tot_eq;
  }
  need_out = need;
  tot_eq_out = tot_eq;
  return prefix;
}

// Mark in `chosen` the k best candidates among the keys this workgroup
// holds.  key[j] is the key of the thread's position j * 1024 + threadIdx.x,
// or 0 if that position is not a candidate.  k must not exceed the number
// of candidates.
//
// Only keys at or above a floor take part in the histograms.  The floor is
// the r-th largest of a sample of four keys per thread (columns spread over
// the row), r set a few standard deviations above the sample rank expected
// for the k-th best; if fewer than k keys reach it, the floor is 1 (every
// candidate).  Either way the k best all lie at or above the floor, so the
// result is the exact one; the sample only decides how much work it takes.
template <int KPT>
__device__ __forceinline__ void reg_select(const uint32_t (&key)[KPT], uint64_t &chosen,
                                           uint32_t k, RegShared<KPT> &sh) {
  if (k == 0) return;
  static_assert(KPT % 4 == 0, "four sample columns per thread");
  const int tid = threadIdx.x, lane = tid % kWave, wave = tid / kWave;
  constexpr int kQ = KPT / 4;
  const int pick = wave % kQ;
  uint32_t smp[4];
#pragma unroll
  for (int s = 0; s < 4; ++s) {
    smp[s] = 0;
#pragma unroll
    for (int q = 0; q < kQ; ++q)
      if (q == pick) smp[s] = key[s * kQ + q];
  }
  uint32_t n_smp;
  block_exclusive_scan((smp[0] != 0u) + (smp[1] != 0u) + (smp[2] != 0u) + (smp[3] != 0u),
                       sh.scan, &n_smp);
  uint32_t floor = 1;
  const float mean = static_cast<float>(k) * (4.f / KPT);
  const uint32_t r = static_cast<uint32_t>(mean + 3.f * sqrtf(mean) + 8.f);
  if (r < n_smp) {
    uint32_t d0, d1;
    const uint32_t e = radix_kth<4, KPT>(smp, 1u, r, sh, d0, d1);
    uint32_t cnt = 0;
#pragma unroll
    for (int j = 0; j < KPT; ++j) cnt += key[j] >= e;
    uint32_t n_above;
    block_exclusive_scan(cnt, sh.scan, &n_above);
    if (n_above >= k) floor = e;
  }
  uint32_t need, tot_eq;
  const uint32_t t = radix_kth<KPT, KPT>(key, floor, k, sh, need, tot_eq);
  // t is the k-th best key (never 0); `need` of the tot_eq keys equal to t
  // are taken, lowest positions first
  uint64_t take = 0, eq = 0;
#pragma unroll
  for (int j = 0; j < KPT; ++j) {
    take |= static_cast<uint64_t>(key[j] > t) << j;
    eq |= static_cast<uint64_t>(key[j] == t) << j;
  }
  if (need == tot_eq) {
    take |= eq;
  } else {
    // position order is (column j, thread)
#pragma unroll
    for (int j = 0; j < KPT; ++j) {
      const uint32_t n = static_cast<uint32_t>(__popcll(__ballot((eq >> j) & 1u)));
      if (lane == 0) sh.colcnt[wave][j] = n;
    }
    __syncthreads();
    if (wave == 0) {
      uint32_t ct = 0;
      if (lane < KPT)
        for (int w = 0; w < kSelWaves; ++w) ct += sh.colcnt[w][lane];
      uint32_t incl = ct;
#pragma unroll
      for (int off = 1; off < kWave; off <<= 1) {
        const uint32_t y = __shfl_up(incl, off, kWave);
        if (lane >= off) incl += y;
      }
      const uint32_t excl = incl - ct;
      if (lane < KPT && excl < need && need <= incl) {
        sh.col_j = static_cast<uint32_t>(lane);
        sh.col_rem = need - excl;
      }
    }
    __syncthreads();
    const int J = min(static_cast<int>(sh.col_j), KPT - 1);
    const uint32_t rem = sh.col_rem;
    uint32_t before = 0;
    for (int w = 0; w < wave; ++w) before += sh.colcnt[w][J];
    const bool eqJ = (eq >> J) & 1u;
    const uint64_t bJ = __ballot(eqJ);
    const uint32_t rank =
        before + static_cast<uint32_t>(__popcll(bJ & ((uint64_t{1} << lane) - 1)));
    take |= eq & ((uint64_t{1} << J) - 1);
    if (eqJ && rank < rem) take |= uint64_t{1} << J;
    __syncthreads();
  }
  chosen |= take;
}

// Word 3 of a gfx9 buffer resource: 32-bit data format, no swizzle.
constexpr int kBufferFlags = 0x00020000;

// key[j] = order key of row[j * 1024 + threadIdx.x] if that position is in
// [lo, hi) (lo < hi) and bit j of `skip` is clear, else 0.
template <int KPT>
__device__ __forceinline__ void load_keys(const float *row, int lo, int hi, uint64_t skip,
                                          uint32_t (&key)[KPT]) {
  const int tid = threadIdx.x;
  // buffer loads: one scalar resource for the row's [0, hi) and a 32-bit
  // byte offset per lane (an offset past the range would read 0)
  const __amdgpu_buffer_rsrc_t rsrc =
      __builtin_amdgcn_make_buffer_rsrc(const_cast<float *>(row), 0, hi * 4, kBufferFlags);
  float v[KPT];
#pragma unroll
  for (int j = 0; j < KPT; ++j) {
    const int q = min(max(j * kSelThreads + tid, lo), hi - 1);
    v[j] = __builtin_bit_cast(float, __builtin_amdgcn_raw_buffer_load_b32(rsrc, q * 4, 0, 0));
  }
  // the loaded values are pinned in registers: without this the compiler
  // moves each load into a branch of its own and waits on it there
#pragma unroll
  for (int j = 0; j < KPT; ++j) asm volatile("" : "+v"(v[j]));
#pragma unroll
  for (int j = 0; j < KPT; ++j) {
    const int p = j * kSelThreads + tid;
    const bool in = p >= lo && p < hi && !((skip >> j) & 1u);
    key[j] = order_key(v[j]) & (in ? ~0u : 0u);
  }
}

template <int KPT>
__global__ __launch_bounds__(kSelThreads) void select_kv_idx_reg(
    const float *draft, const float *target, int score_len, const int32_t *ctx_lens, int hkv,
    int n_sel, int n_sink, int n_recent, int n_draft_top, int32_t *kv_idx) {
  static_assert(KPT >= 1 && KPT <= 64, "one 64-bit mask per thread");
  __shared__ RegShared<KPT> sh;
  const int tid = threadIdx.x, lane = tid % kWave, wave = tid / kWave;
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

  const int64_t row0 = static_cast<int64_t>(bg) * score_len;
  uint64_t chosen = 0;
  uint32_t key[KPT];
  // Every load is unconditional, from a position clamped into the candidate
  // range [lo, hi) (non-empty whenever m or rest is positive), so the
  // compiler issues all KPT loads before the first wait; non-candidates then
  // get key 0.
  if (m > 0) {
    load_keys<KPT>(draft + row0, lo, hi, 0, key);
    reg_select<KPT>(key, chosen, static_cast<uint32_t>(m), sh);
  }
  if (rest > 0) {
    load_keys<KPT>(target + row0, lo, hi, chosen, key);
    reg_select<KPT>(key, chosen, static_cast<uint32_t>(rest), sh);
  }

  // bitmap entry j * 16 + wave covers positions j * 1024 + 64 * wave + [0, 64)
#pragma unroll
  for (int j = 0; j < KPT; ++j) {
    const int p = j * kSelThreads + tid;
    const bool in = ((chosen >> j) & 1u) || (p < c && (p < lo || p >= hi));
    const uint64_t bj = __ballot(in);
    if (lane == 0) sh.bitmap[j * kSelWaves + wave] = bj;
  }
  __syncthreads();

  // ascending compaction: thread t owns entry t
  constexpr int kEntries = KPT * kSelWaves;
  const uint64_t v0 = tid < kEntries ? sh.bitmap[tid] : 0;
  uint32_t total;
  uint32_t out = block_exclusive_scan(static_cast<uint32_t>(__popcll(v0)), sh.scan, &total);
  int32_t *dst = kv_idx + static_cast<int64_t>(bg) * n_sel;
  uint64_t v = v0;
  while (v) {
    const int j = __ffsll(static_cast<unsigned long long>(v)) - 1;
    v &= v - 1;
    if (out < static_cast<uint32_t>(n_sel)) dst[out] = 64 * tid + j;
    ++out;
  }
  for (int s = static_cast<int>(total) + tid; s < n_sel; s += kSelThreads) dst[s] = -1;
}

}  // namespace

int select_max_positions() { return 1 << 19; }

hipError_t launch_select_kv_idx(const float *draft, const float *target, int score_len,
                                const int32_t *ctx_lens, int batch, int hkv, int n_sel,
                                int n_sink, int n_recent, int n_draft_top, int32_t *kv_idx,
                                hipStream_t s) {
  const dim3 grid(static_cast<unsigned>(batch * hkv)), block(kSelThreads);
  if (score_len <= 16 * kSelThreads) {
    hipLaunchKernelGGL(select_kv_idx_reg<16>, grid, block, 0, s, draft, target, score_len,
                       ctx_lens, hkv, n_sel, n_sink, n_recent, n_draft_top, kv_idx);
  } else if (score_len <= 32 * kSelThreads) {
    hipLaunchKernelGGL(select_kv_idx_reg<32>, grid, block, 0, s, draft, target, score_len,
                       ctx_lens, hkv, n_sel, n_sink, n_recent, n_draft_top, kv_idx);
  } else if (score_len <= 64 * kSelThreads) {
    hipLaunchKernelGGL(select_kv_idx_reg<64>, grid, block, 0, s, draft, target, score_len,
                       ctx_lens, hkv, n_sel, n_sink, n_recent, n_draft_top, kv_idx);
  } else {
    const size_t lds = static_cast<size_t>((score_len + 31) / 32) * sizeof(uint32_t);
    hipLaunchKernelGGL(select_kv_idx_stream, grid, block, lds, s, draft, target, score_len,
                       ctx_lens, hkv, n_sel, n_sink, n_recent, n_draft_top, kv_idx);
  }
  return hipGetLastError();
}

}  // namespace hsv
