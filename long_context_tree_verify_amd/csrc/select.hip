// Verification index-set selection (Dustin page, methodology 1: hybrid
// attention aggregation; verification workflow step 3 forms the compressed
// cache from these positions).
//
// Per (sequence b, KV head g), of the positions [0, c): the first n_sink and
// the last n_recent are kept; of the middle ones (the candidates), the m best
// by the draft-lookahead score, then the best remaining ones by the
// target-historical score until n_sel are chosen.  "Best": higher score, NaN
// below every number, -0 equal to +0, ties to the lower position.  The
// chosen positions are marked in an LDS bitmap and written out ascending; if
// fewer than n_sel exist the tail is -1.
//
// Scores become order-preserving 32-bit keys; with the position appended
// (key, then the position inverted) every candidate has a distinct value and
// "the k best" is "every value at or above the k-th largest".
//
// Two launches:
//  1. select_filter (one 256-thread workgroup per 8192-position chunk of a
//     row, so every CU streams): from a fixed sample of the row (32 spread
//     segments of 64 positions) the workgroup finds a floor key for each map
//     -- the 22-bit prefix of the sample's r-th largest key, r a few standard
//     deviations above the rank the k-th best would have in the sample -- and
//     appends the (key, position) pairs of its chunk at or above the floor to
//     its own slots in the workspace.  Every chunk of a row derives the same
//     floors from the same sample.
//  2. select_lists (one 1024-thread workgroup per row): loads a map's short
//     list into LDS and runs an exact radix select over (key, position).  The
//     list answers the question whenever at least k listed candidates remain
//     (for the target: once the draft's picks are removed): then the k-th
//     best is at or above the floor, and every candidate at or above the
//     floor was listed.  Otherwise (or if a list overflowed) that map falls
//     back to a streaming radix select over the whole row.  Either way the
//     result is the exact one.
// Both kernels are short loops: the selection is instruction-fetch bound if
// its code is unrolled over a row held in registers.
#include "common.hpp"
#include "launch.h"

namespace hsv {
namespace {

constexpr int kSelThreads = 1024;
constexpr int kSelWaves = kSelThreads / kWave;
constexpr int kFiltThreads = 256;
constexpr int kChunk = 8192;        // positions per filter workgroup
constexpr int kChunkCap = 1024;     // list slots per (chunk, map)
constexpr int kListCap = 8192;      // list entries a row's select holds in LDS
constexpr int kMaxChunks = 64;      // rows of up to 2^19 positions
constexpr int kSegs = 32, kSegLen = 64, kSample = kSegs * kSegLen;
constexpr int kBins = 2048;         // 11-bit digits
constexpr int kPosBits = 19;        // positions < 2^19
constexpr int kBufferFlags = 0x00020000;  // word 3 of a gfx9 buffer resource: 32-bit data

// Order-preserving key: larger score -> larger key; NaN -> 1 (below every
// number, -inf included); -0 -> the key of +0.  No score maps to 0, which
// marks "not a candidate".
__device__ __forceinline__ uint32_t order_key(float f) {
  if (f != f) return 1u;
  uint32_t u = __float_as_uint(f == 0.f ? 0.f : f);
  return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}

// The budget split of one sequence (the same arithmetic in both kernels).
struct Budget {
  int c, lo, hi, m, rest;
};
__device__ __forceinline__ Budget budget(int ctx, int score_len, int n_sel, int n_sink,
                                         int n_recent, int n_draft_top) {
  Budget bd;
  bd.c = min(max(ctx, 0), score_len);
  bd.lo = min(n_sink, bd.c);
  bd.hi = max(bd.c - n_recent, bd.lo);
  const int n_protected = bd.lo + (bd.c - bd.hi);
  const int fill = n_sel - n_protected;
  const int n_cand = bd.hi - bd.lo;
  bd.m = min(min(n_draft_top, fill), n_cand);
  bd.rest = min(fill - bd.m, n_cand - bd.m);
  return bd;
}

// Inclusive prefix sum over the 64 lanes of a wave: DPP row shifts by 1, 2,
// 4 and 8 scan each 16-lane row, then row broadcasts of lanes 15 and 31 carry
// the row totals forward (lanes a DPP move does not write read 0).
__device__ __forceinline__ uint32_t wave_inclusive_scan(uint32_t x) {
  int v = static_cast<int>(x);
  v += __builtin_amdgcn_update_dpp(0, v, 0x111, 0xf, 0xf, false);  // row_shr:1
  v += __builtin_amdgcn_update_dpp(0, v, 0x112, 0xf, 0xf, false);  // row_shr:2
  v += __builtin_amdgcn_update_dpp(0, v, 0x114, 0xf, 0xf, false);  // row_shr:4
  v += __builtin_amdgcn_update_dpp(0, v, 0x118, 0xf, 0xf, false);  // row_shr:8
  v += __builtin_amdgcn_update_dpp(0, v, 0x142, 0xa, 0xf, false);  // row_bcast:15
  v += __builtin_amdgcn_update_dpp(0, v, 0x143, 0xc, 0xf, false);  // row_bcast:31
  return static_cast<uint32_t>(v);
}

// Exclusive prefix sum of `x` over a workgroup of NT threads, in thread
// order; `total` receives the sum.  Uses `scratch` (NT / 64 words).
template <int NT>
__device__ __forceinline__ uint32_t block_exclusive_scan(uint32_t x, uint32_t *scratch,
                                                         uint32_t *total) {
  constexpr int kW = NT / kWave;
  const int lane = threadIdx.x % kWave, wave = threadIdx.x / kWave;
  const uint32_t incl = wave_inclusive_scan(x);
  if (lane == kWave - 1) scratch[wave] = incl;
  __syncthreads();
  uint32_t wave_base = 0, all = 0;
#pragma unroll
  for (int w = 0; w < kW; ++w) {
    const uint32_t s = scratch[w];
    if (w < wave) wave_base += s;
    all += s;
  }
  __syncthreads();
  *total = all;
  return wave_base + incl - x;
}

// Digit search over a histogram of kBins counts (bin-major, COPIES
// interleaved copies): the bin holding the need-th largest value.  Thread t
// owns kBins/NT bins from kBins-1-(kBins/NT)*t downwards, so thread order is
// descending bin order.  The one thread whose bin holds it writes *digit,
// *need_out (the rank inside the bin) and *in_bin (the bin's count); the
// caller then meets at a barrier.  The histogram must hold at least `need`.
// Each thread zeroes the bins it read, so after that barrier the histogram
// is clear for the next pass.
template <int NT, int COPIES>
__device__ __forceinline__ void find_digit(uint32_t *hist, uint32_t need, uint32_t *scan,
                                           uint32_t *digit, uint32_t *need_out,
                                           uint32_t *in_bin) {
  constexpr int kPer = kBins / NT;
  const int top = kBins - 1 - kPer * static_cast<int>(threadIdx.x);
  uint32_t cnt[kPer];
  uint32_t mine = 0;
#pragma unroll
  for (int i = 0; i < kPer; ++i) {
    uint32_t s = 0;
#pragma unroll
    for (int cp = 0; cp < COPIES; ++cp) {
      s += hist[(top - i) * COPIES + cp];
      hist[(top - i) * COPIES + cp] = 0u;
    }
    cnt[i] = s;
    mine += s;
  }
  uint32_t total;
  uint32_t above = block_exclusive_scan<NT>(mine, scan, &total);
#pragma unroll
  for (int i = 0; i < kPer; ++i) {
    if (above < need && need <= above + cnt[i]) {
      *digit = static_cast<uint32_t>(top - i);
      *need_out = need - above;
      *in_bin = cnt[i];
    }
    above += cnt[i];
  }
}

// ---------------------------------------------------------------------------
// Streaming radix select (the fallback): mark the k best candidates of
// row[lo, hi) that are not yet in `bits`.  Four 8-bit passes read the row
// (from L2 after the first); ties at the k-th key are ranked chunk by chunk.
// ---------------------------------------------------------------------------
struct StreamShared {
  uint32_t hist[kSelWaves][256];
  uint32_t tot[256];
  uint32_t scan[kSelWaves];
  uint32_t digit, need;
};

__device__ void select_best(const float *row, int lo, int hi, uint32_t k, uint32_t *bits,
                            StreamShared &sh) {
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
    const uint32_t rank = block_exclusive_scan<kSelThreads>(eq ? 1u : 0u, sh.scan, &n_eq);
    if (gt || (eq && taken_eq + rank < need)) atomicOr(&bits[p >> 5], 1u << (p & 31));
    taken_eq += n_eq;
    __syncthreads();
  }
  __syncthreads();
}

// ---------------------------------------------------------------------------
// Filter: floors from the sample, then the chunk's candidates at or above
// them appended to the chunk's list slots.
// ---------------------------------------------------------------------------
struct FiltShared {
  uint4 keys4[kChunk / 4];          // the chunk's keys
  uint32_t hist[kBins];
  uint32_t scan[kFiltThreads / kWave];
  uint32_t digit, need, in_bin, n_out;
};

// i-th sample position of a row whose candidates are [lo, lo + n_cand):
// all of them when there are at most kSample, else 32 segments of 64
// consecutive positions spread evenly.
__device__ __forceinline__ int sample_pos(int i, int lo, int n_cand) {
  if (n_cand <= kSample) return lo + i;
  const int s = i / kSegLen;
  return lo + static_cast<int>(static_cast<int64_t>(n_cand - kSegLen) * s / (kSegs - 1)) +
         i % kSegLen;
}

// Floor key for "the k best of n_cand candidates": the smallest key sharing
// its top 22 bits with the r-th largest sample key, or 1 (every candidate)
// when the sample is too small for r.
__device__ uint32_t sample_floor(const float *row, int lo, int n_cand, int k, FiltShared &sh) {
  const int tid = threadIdx.x;
  const int n_smp = min(n_cand, kSample);
  const float mean = static_cast<float>(k) * n_smp / n_cand;
  const uint32_t r = static_cast<uint32_t>(ceilf(mean + 3.f * sqrtf(mean) + 8.f));
  if (r >= static_cast<uint32_t>(n_smp)) return 1u;
  constexpr int kPer = kSample / kFiltThreads;
  float v[kPer];
#pragma unroll
  for (int u = 0; u < kPer; ++u)  // unconditional: all loads in flight together
    v[u] = row[sample_pos(min(tid + kFiltThreads * u, n_smp - 1), lo, n_cand)];
  uint32_t key[kPer];
#pragma unroll
  for (int u = 0; u < kPer; ++u) key[u] = tid + kFiltThreads * u < n_smp ? order_key(v[u]) : 0u;
  uint32_t prefix = 0, pmask = 0, need = r;
  for (int i = tid; i < kBins; i += kFiltThreads) sh.hist[i] = 0u;
  __syncthreads();
#pragma unroll
  for (int pass = 0; pass < 2; ++pass) {
    const int shift = pass == 0 ? 21 : 10;
#pragma unroll
    for (int u = 0; u < kPer; ++u)
      if (key[u] != 0u && (key[u] & pmask) == prefix)
        atomicAdd(&sh.hist[(key[u] >> shift) & (kBins - 1)], 1u);
    __syncthreads();
    find_digit<kFiltThreads, 1>(sh.hist, need, sh.scan, &sh.digit, &sh.need, &sh.in_bin);
    __syncthreads();
    prefix |= sh.digit << shift;
    pmask |= static_cast<uint32_t>(kBins - 1) << shift;
    need = sh.need;
  }
  __syncthreads();  // sh.digit / sh.need are read before anyone rewrites them
  return max(prefix, 1u);
}

__global__ __launch_bounds__(kFiltThreads) void select_filter_kernel(
    const float *draft, const float *target, int score_len, const int32_t *ctx_lens, int hkv,
    int n_sel, int n_sink, int n_recent, int n_draft_top, int nch, uint32_t *counts,
    uint2 *lists) {
  __shared__ FiltShared sh;
  const int tid = threadIdx.x, lane = tid % kWave;
  const int bg = blockIdx.x / nch, ch = blockIdx.x % nch;
  const Budget bd = budget(ctx_lens[bg / hkv], score_len, n_sel, n_sink, n_recent, n_draft_top);
  const int n_cand = bd.hi - bd.lo;
  const int64_t row0 = static_cast<int64_t>(bg) * score_len;
  const int p_begin = max(ch * kChunk, bd.lo), p_end = min(ch * kChunk + kChunk, bd.hi);
#pragma unroll 1
  for (int map = 0; map < 2; ++map) {
    const int k = map == 0 ? bd.m : min(bd.rest + bd.m, n_cand);
    uint32_t *count = counts + (static_cast<int64_t>(bg) * nch + ch) * 2 + map;
    uint2 *list = lists + ((static_cast<int64_t>(bg) * nch + ch) * 2 + map) * kChunkCap;
    if (k <= 0 || p_end <= p_begin) {
      if (tid == 0) *count = 0;
      continue;
    }
    const float *row = (map == 0 ? draft : target) + row0;
    const uint32_t floor = sample_floor(row, bd.lo, n_cand, k, sh);
    // Stage the chunk's keys (0 outside [p_begin, p_end)): positions
    // ch*8192 + 4*(tid + 256 u) + e, each thread's eight 16-byte buffer
    // loads issued unconditionally (dword alignment suffices; a load that
    // would pass hi is moved back to end at hi, so nothing at or past hi --
    // hence c -- is read).  A quad that crosses hi is staged as 0 here; its
    // at most three candidates are appended after the loop.
    constexpr int kU = kChunk / (4 * kFiltThreads);
    if (bd.hi >= 4) {
      const __amdgpu_buffer_rsrc_t rsrc = __builtin_amdgcn_make_buffer_rsrc(
          const_cast<float *>(row), 0, bd.hi * 4, kBufferFlags);
      uint32_t x[kU][4];
#pragma unroll
      for (int u = 0; u < kU; ++u) {
        const int p4 = ch * kChunk + 4 * (tid + kFiltThreads * u);
        const auto q = __builtin_amdgcn_raw_buffer_load_b128(rsrc, min(p4, bd.hi - 4) * 4, 0, 0);
        x[u][0] = q[0], x[u][1] = q[1], x[u][2] = q[2], x[u][3] = q[3];
      }
#pragma unroll
      for (int u = 0; u < kU; ++u) {
        const int p4 = ch * kChunk + 4 * (tid + kFiltThreads * u);
        const bool whole = p4 + 3 < bd.hi;
        uint32_t kk[4];
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const int p = p4 + e;
          kk[e] = (whole && p >= p_begin && p < p_end) ? order_key(__uint_as_float(x[u][e])) : 0u;
        }
        sh.keys4[tid + kFiltThreads * u] = make_uint4(kk[0], kk[1], kk[2], kk[3]);
      }
    } else {
      for (int u = tid; u < kChunk / 4; u += kFiltThreads) sh.keys4[u] = make_uint4(0, 0, 0, 0);
    }
    if (tid == 0) sh.n_out = 0;
    __syncthreads();
    // append the keys at or above the floor (key 0 never is): each wave
    // counts its survivors, reserves them with one LDS atomic, then writes
    // them in (u, e, lane) order
    uint4 kq[kU];
    uint32_t n_keep = 0;
#pragma unroll
    for (int u = 0; u < kU; ++u) {
      kq[u] = sh.keys4[tid + kFiltThreads * u];
      n_keep += __popcll(__ballot(kq[u].x >= floor)) + __popcll(__ballot(kq[u].y >= floor)) +
                __popcll(__ballot(kq[u].z >= floor)) + __popcll(__ballot(kq[u].w >= floor));
    }
    uint32_t base = 0;
    if (lane == 0 && n_keep) base = atomicAdd(&sh.n_out, n_keep);
    base = __shfl(base, 0, kWave);
    const uint64_t below = (uint64_t{1} << lane) - 1;
#pragma unroll
    for (int u = 0; u < kU; ++u) {
      const int p4 = ch * kChunk + 4 * (tid + kFiltThreads * u);
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const uint32_t key = e == 0 ? kq[u].x : e == 1 ? kq[u].y : e == 2 ? kq[u].z : kq[u].w;
        const bool keep = key >= floor;
        const uint64_t bal = __ballot(keep);
        if (keep) {
          const uint32_t slot = base + static_cast<uint32_t>(__popcll(bal & below));
          if (slot < static_cast<uint32_t>(kChunkCap)) list[slot] = make_uint2(key, p4 + e);
        }
        base += static_cast<uint32_t>(__popcll(bal));
      }
    }
    // the quad that crosses hi (or, for hi < 4, the whole range): single loads
    {
      const int t0 = bd.hi >= 4 ? (bd.hi & ~3) : 0;
      const int p = t0 + tid;
      if (tid < 4 && p < bd.hi && p >= p_begin && p < p_end) {
        const uint32_t key = order_key(row[p]);
        if (key >= floor) {
          const uint32_t slot = atomicAdd(&sh.n_out, 1u);
          if (slot < static_cast<uint32_t>(kChunkCap)) list[slot] = make_uint2(key, p);
        }
      }
    }
    __syncthreads();
    if (tid == 0) *count = sh.n_out;
    __syncthreads();
  }
}

// ---------------------------------------------------------------------------
// Per-row select over the lists, the fallback, and the write-out.
// ---------------------------------------------------------------------------
struct ListShared {
  union {
    StreamShared stream;            // fallback; its histogram doubles as the list's
    uint32_t hist2[kBins * 2];      // list histogram, 2 interleaved copies
  };
  int32_t out_stage[kListCap];      // the sorted set, written out coalesced
  uint32_t cnt[kMaxChunks];
  uint32_t scan[kSelWaves];
  uint32_t digit, need, in_bin, ok;
};

// Select the k best (k >= 1) of map `map`'s list into `bits`; false (and
// nothing marked) if the list cannot answer (see the file comment).  Rows of
// up to kListCap / kChunkCap chunks only: thread t holds slot t of every
// chunk's list in registers (slots past a chunk's count hold key 0), all
// loaded in one batch.
__device__ bool list_select(const uint32_t *counts, const uint2 *lists, int bg, int nch, int map,
                            uint32_t k, uint32_t *bits, ListShared &sh) {
  constexpr int kMaxListChunks = kListCap / kChunkCap;
  static_assert(kChunkCap == kSelThreads, "one slot per thread and chunk");
  const int tid = threadIdx.x, lane = tid % kWave;
  if (nch > kMaxListChunks) return false;
  if (tid < kWave) {
    const uint32_t n =
        lane < nch ? counts[(static_cast<int64_t>(bg) * nch + lane) * 2 + map] : 0u;
    const bool over = __any(n > static_cast<uint32_t>(kChunkCap));
    uint32_t sum = n;
#pragma unroll
    for (int o = 32; o >= 1; o >>= 1) sum += __shfl_xor(sum, o, kWave);
    if (lane < nch) sh.cnt[lane] = n;
    if (lane == 0) sh.ok = !over && sum >= k;
  }
  __syncthreads();
  if (!sh.ok) return false;
  // all slots of all chunks, loads in flight together (chunks past nch read
  // the last chunk's slots and are dropped); each thread keeps slot tid of
  // every chunk in registers.  Positions already chosen (the draft's picks,
  // for the target) get key 0.
  const uint2 *src = lists + (static_cast<int64_t>(bg) * nch * 2 + map) * kChunkCap + tid;
  uint2 e[kMaxListChunks];
#pragma unroll
  for (int u = 0; u < kMaxListChunks; ++u)
    e[u] = src[static_cast<int64_t>(min(u, nch - 1)) * 2 * kChunkCap];
  uint32_t valid = 0;
#pragma unroll
  for (int u = 0; u < kMaxListChunks; ++u) {
    if (u >= nch || static_cast<uint32_t>(tid) >= sh.cnt[u] ||
        ((bits[e[u].y >> 5] >> (e[u].y & 31)) & 1u))
      e[u].x = 0u;
    valid += e[u].x != 0u;
  }
  uint32_t n_valid;
  block_exclusive_scan<kSelThreads>(valid, sh.scan, &n_valid);
  if (n_valid < k) return false;

  // radix select over value = (key << 19) | (2^19 - 1 - position): passes of
  // 11/11/10 key bits, then 11/8 position bits if the k-th key is shared
  constexpr uint32_t kPosMask = (1u << kPosBits) - 1;
  const uint32_t copy = static_cast<uint32_t>(lane) & 1u;
  uint32_t kpre = 0, kmask = 0, ppre = 0, pmask = 0, need = k, in_bin = 0;
  for (int i = tid; i < kBins * 2; i += kSelThreads) sh.hist2[i] = 0u;
  __syncthreads();
  for (int pass = 0; pass < 5; ++pass) {
    if (pass == 3 && need == in_bin) break;  // every key equal to the k-th is taken
    const bool on_pos = pass >= 3;
    const int shift = pass == 0 ? 21 : pass == 1 ? 10 : pass == 3 ? 8 : 0;
    const uint32_t dmask = pass == 2 ? 1023u : pass == 4 ? 255u : 2047u;
#pragma unroll
    for (int u = 0; u < kMaxListChunks; ++u) {
      const uint32_t inv = kPosMask - e[u].y;
      if (e[u].x != 0u && (e[u].x & kmask) == kpre && (inv & pmask) == ppre) {
        const uint32_t d = ((on_pos ? inv : e[u].x) >> shift) & dmask;
        atomicAdd(&sh.hist2[d * 2 + copy], 1u);
      }
    }
    __syncthreads();
    find_digit<kSelThreads, 2>(sh.hist2, need, sh.scan, &sh.digit, &sh.need, &sh.in_bin);
    __syncthreads();
    if (on_pos) {
      ppre |= sh.digit << shift;
      pmask |= dmask << shift;
    } else {
      kpre |= sh.digit << shift;
      kmask |= dmask << shift;
    }
    need = sh.need;
    in_bin = sh.in_bin;
  }
  __syncthreads();  // sh.digit / sh.need are read before anyone rewrites them
  // mark every value at or above the k-th: key above it, or equal key and
  // (when positions were resolved) position at or before it
#pragma unroll
  for (int u = 0; u < kMaxListChunks; ++u) {
    const uint32_t inv = kPosMask - e[u].y;
    const bool take =
        e[u].x != 0u && (e[u].x > kpre || (e[u].x == kpre && (pmask == 0 || inv >= ppre)));
    if (take) atomicOr(&bits[e[u].y >> 5], 1u << (e[u].y & 31));
  }
  __syncthreads();
  return true;
}

// Bits of positions [a, b) that fall in the word of positions [p0, p0 + 32).
__device__ __forceinline__ uint32_t range_bits(int p0, int a, int b) {
  const int lo = max(a - p0, 0), hi = min(b - p0, 32);
  if (lo >= hi) return 0u;
  const uint32_t upto = hi == 32 ? ~0u : ((1u << hi) - 1u);
  return upto & ~((1u << lo) - 1u);
}

__global__ __launch_bounds__(kSelThreads) void select_lists_kernel(
    const float *draft, const float *target, int score_len, const int32_t *ctx_lens, int hkv,
    int n_sel, int n_sink, int n_recent, int n_draft_top, int nch, const uint32_t *counts,
    const uint2 *lists, int32_t *kv_idx) {
  extern __shared__ uint32_t bits[];  // ceil(score_len / 32) words
  __shared__ ListShared sh;
  const int tid = threadIdx.x;
  const int bg = blockIdx.x;
  const Budget bd = budget(ctx_lens[bg / hkv], score_len, n_sel, n_sink, n_recent, n_draft_top);

  const int words = (bd.c + 31) / 32;
  for (int w = tid; w < words; w += kSelThreads) {
    // protected positions: [0, lo) and [hi, c)
    bits[w] = range_bits(32 * w, 0, bd.lo) | range_bits(32 * w, bd.hi, bd.c);
  }
  __syncthreads();

  const int64_t row0 = static_cast<int64_t>(bg) * score_len;
  if (bd.m > 0 &&
      !list_select(counts, lists, bg, nch, 0, static_cast<uint32_t>(bd.m), bits, sh))
    select_best(draft + row0, bd.lo, bd.hi, static_cast<uint32_t>(bd.m), bits, sh.stream);
  if (bd.rest > 0 &&
      !list_select(counts, lists, bg, nch, 1, static_cast<uint32_t>(bd.rest), bits, sh))
    select_best(target + row0, bd.lo, bd.hi, static_cast<uint32_t>(bd.rest), bits, sh.stream);

  // ascending compaction: thread t owns a contiguous run of words; sets that
  // fit are staged in LDS and written out coalesced, with the -1 tail
  const int per = (words + kSelThreads - 1) / kSelThreads;
  const int w0 = min(tid * per, words), w1 = min(w0 + per, words);
  uint32_t cnt = 0;
  for (int w = w0; w < w1; ++w) cnt += __popc(bits[w]);
  uint32_t total;
  uint32_t out = block_exclusive_scan<kSelThreads>(cnt, sh.scan, &total);
  int32_t *dst = kv_idx + static_cast<int64_t>(bg) * n_sel;
  const bool staged = n_sel <= kListCap;
  for (int w = w0; w < w1; ++w) {
    const uint32_t v = bits[w];
    if (staged) {
#pragma unroll
      for (int j = 0; j < 32; ++j) {
        const uint32_t at = out + static_cast<uint32_t>(__popc(v & ((1u << j) - 1u)));
        if (((v >> j) & 1u) && at < static_cast<uint32_t>(n_sel)) sh.out_stage[at] = 32 * w + j;
      }
      out += static_cast<uint32_t>(__popc(v));
    } else {
      uint32_t r = v;
      while (r) {
        const int j = __ffs(r) - 1;
        r &= r - 1;
        if (out < static_cast<uint32_t>(n_sel)) dst[out] = 32 * w + j;
        ++out;
      }
    }
  }
  if (staged) {
    __syncthreads();
    for (int s = tid; s < n_sel; s += kSelThreads)
      dst[s] = s < static_cast<int>(total) ? sh.out_stage[s] : -1;
  } else {
    for (int s = static_cast<int>(total) + tid; s < n_sel; s += kSelThreads) dst[s] = -1;
  }
}

int select_chunks(int score_len) { return (score_len + kChunk - 1) / kChunk; }

size_t select_count_bytes(size_t rows, int nch) {
  return (rows * static_cast<size_t>(nch) * 2 * sizeof(uint32_t) + 255) / 256 * 256;
}

}  // namespace

int select_max_positions() { return 1 << kPosBits; }

size_t select_workspace_bytes(int batch, int hkv, int score_len) {
  const size_t rows = static_cast<size_t>(batch) * hkv;
  const int nch = select_chunks(score_len);
  return select_count_bytes(rows, nch) +
         rows * static_cast<size_t>(nch) * 2 * kChunkCap * sizeof(uint2);
}

hipError_t launch_select_kv_idx(const float *draft, const float *target, int score_len,
                                const int32_t *ctx_lens, int batch, int hkv, int n_sel,
                                int n_sink, int n_recent, int n_draft_top, int32_t *kv_idx,
                                void *workspace, hipStream_t s) {
  const int nch = select_chunks(score_len);
  if (nch > kMaxChunks) return hipErrorInvalidValue;
  const size_t rows = static_cast<size_t>(batch) * hkv;
  uint32_t *counts = static_cast<uint32_t *>(workspace);
  uint2 *lists = reinterpret_cast<uint2 *>(static_cast<char *>(workspace) +
                                           select_count_bytes(rows, nch));
  hipLaunchKernelGGL(select_filter_kernel, dim3(static_cast<unsigned>(rows * nch)),
                     dim3(kFiltThreads), 0, s, draft, target, score_len, ctx_lens, hkv, n_sel,
                     n_sink, n_recent, n_draft_top, nch, counts, lists);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  const size_t lds = static_cast<size_t>((score_len + 31) / 32) * sizeof(uint32_t);
  hipLaunchKernelGGL(select_lists_kernel, dim3(static_cast<unsigned>(rows)), dim3(kSelThreads),
                     lds, s, draft, target, score_len, ctx_lens, hkv, n_sel, n_sink, n_recent,
                     n_draft_top, nch, counts, lists, kv_idx);
  return hipGetLastError();
}

}  // namespace hsv
