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
// Rows of up to 73728 positions (a 64k context and its draft rows) take
// three launches, each a short chain of memory round trips:
//  1. select_floor (one 1024-thread workgroup per row): from a fixed sample
//     of the row (32 segments of 64 positions spread over it; those inside
//     the candidate range count) each map gets a floor key -- the 22-bit
//     prefix of the sample's r-th largest key, r a few standard deviations
//     above the rank the k-th best would have in the sample -- in two radix
//     passes that serve both maps.
//  2. select_filter (one 256-thread workgroup per 8192-position chunk of a
//     row, both maps at once, so every CU streams): the floor becomes the
//     smallest score whose key is at or above it, so the chunk is tested
//     with one float compare per score; the scores that pass (raw bits and
//     position) are appended to the chunk's own slots in the workspace.
//  3. select_lists (one 1024-thread workgroup per row): every list slot of
//     both maps is loaded at once and stays in registers.  One pass counts
//     both maps' listed keys into floor-relative histograms (the draft's
//     picks leave the target's once they are known); the first digit then
//     names the bin of the k-th value, whose few entries are ranked
//     directly, or the radix passes take key bits 10..20 and 0..9 (skipped
//     when every entry left shares them) and the few entries left sharing
//     the k-th key are ranked by position.  A list answers the question whenever at
//     least k listed candidates remain: then the k-th best is at or above
//     the floor, and every candidate at or above the floor was listed.
//     Otherwise (or if a list overflowed, or candidates lie past the first
//     65536 positions, which have no list slots) that map falls back to a
//     streaming radix select over the row.  Either way the result is the
//     exact one.
//     Sinks and window go to their known output slots, the picked candidates
//     to theirs by a prefix sum of bitmap popcounts, written straight out.
// Longer rows take select_stream: the streaming select for both maps.
// Scores at or past c do not affect the result (the kernels read the rows
// without waiting for the context lengths, and drop those positions).
#include "common.hpp"
#include "launch.h"

namespace hsv {
namespace {

constexpr int kSelThreads = 1024;
constexpr int kSelWaves = kSelThreads / kWave;
constexpr int kFiltThreads = 256;
constexpr int kChunk = 8192;          // positions per filter workgroup
constexpr int kQuads = kChunk / (4 * kFiltThreads);  // 16-byte loads per thread and map
constexpr int kChunkCap = 1024;       // list slots per (chunk, map)
constexpr int kListChunks = 8;        // rows of up to 8 chunks take the list path
constexpr int kListMax = kListChunks * kChunk;  // 65536 positions with list slots
constexpr int kBitsMax = kListMax + kChunk;     // rows the list path takes (a 64k context plus
                                                // its draft rows); entries past kListMax go to
                                                // the streaming fallback
constexpr int kWords = kBitsMax / 32;
constexpr int kTieCap = 256;          // entries sharing the k-th key ranked directly
constexpr int kRankCap = 256;         // entries of the k-th value's floor-relative bin ranked directly
constexpr int kSegs = 32, kSegLen = 64, kSample = kSegs * kSegLen;
constexpr int kSmpPer = kSample / kSelThreads;
constexpr int kBins = 2048;           // 11-bit digits
constexpr int kCopies = 1;            // copies of the first-digit histogram (the fallback
                                      // bins could take interleaved ones)
constexpr int kPosBits = 19;          // positions < 2^19
constexpr uint32_t kPosMask = (1u << kPosBits) - 1;
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
// order; `total` receives the sum.  Uses `scratch` (NT / 64 words).  With
// TAIL the call ends with a barrier, so it may be called again at once;
// without, the caller must pass a barrier before `scratch` is reused.
template <int NT, bool TAIL = true>
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
  if (TAIL) __syncthreads();
  *total = all;
  return wave_base + incl - x;
}

// Where bin b (copy cp) of a histogram with COPIES interleaved copies lives.
template <int COPIES = 1>
__device__ __forceinline__ int hslot(uint32_t b, uint32_t cp = 0) {
  return static_cast<int>(b * COPIES + cp);
}

// Digit search over a histogram of kBins counts (COPIES interleaved
// copies): the bin holding the need-th largest value.  Thread t
// owns kBins/NT bins from kBins-1-(kBins/NT)*t downwards, so thread order is
// descending bin order.  The one thread whose bin holds it writes *digit,
// *need_out (the rank inside the bin) and *in_bin (the bin's count); no
// thread does if the histogram holds fewer than `need`.  Returns the
// histogram's total to every thread.  Each thread zeroes the bins it read.
// The caller passes a barrier before reading the outputs and before the
// next call (the scan scratch is reused).
template <int NT, int COPIES>
__device__ __forceinline__ uint32_t find_digit(uint32_t *hist, uint32_t need, uint32_t *scan,
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
      const int a = hslot<COPIES>(static_cast<uint32_t>(top - i), static_cast<uint32_t>(cp));
      s += hist[a];
      hist[a] = 0u;
    }
    cnt[i] = s;
    mine += s;
  }
  uint32_t total;
  uint32_t above = block_exclusive_scan<NT, false>(mine, scan, &total);
#pragma unroll
  for (int i = 0; i < kPer; ++i) {
    if (above < need && need <= above + cnt[i]) {
      *digit = static_cast<uint32_t>(top - i);
      *need_out = need - above;
      *in_bin = cnt[i];
    }
    above += cnt[i];
  }
  return total;
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

__device__ __forceinline__ void select_best(const float *row, int lo, int hi, uint32_t k, uint32_t *bits,
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
// The sample: 32 segments of 64 consecutive positions spread evenly over the
// row (all positions when it has at most kSample); only those inside the
// candidate range count.
// ---------------------------------------------------------------------------
__device__ __forceinline__ int segment_start(int s, int score_len) {
  return (score_len - kSegLen) * s / (kSegs - 1);  // < 2^19 * 31: no overflow
}
__device__ __forceinline__ int sample_pos(int i, int score_len) {
  if (score_len <= kSample) return i;
  return segment_start(i / kSegLen, score_len) + i % kSegLen;
}
// (Lane s of every wave takes segment s; a wave sum adds them up.)
__device__ __forceinline__ int sample_in_range(int lo, int hi, int score_len) {
  if (score_len <= kSample) return max(hi - lo, 0);
  const int s = static_cast<int>(threadIdx.x % kWave);
  const int a = segment_start(s, score_len);
  int n = s < kSegs ? max(0, min(a + kSegLen, hi) - max(a, lo)) : 0;
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) n += __shfl_xor(n, o, kWave);
  return n;
}

// Bits of positions [a, b) that fall in the word of positions [p0, p0 + 32).
__device__ __forceinline__ uint32_t range_bits(int p0, int a, int b) {
  const int lo = max(a - p0, 0), hi = min(b - p0, 32);
  if (lo >= hi) return 0u;
  const uint32_t upto = hi == 32 ? ~0u : ((1u << hi) - 1u);
  return upto & ~((1u << lo) - 1u);
}

// The select's state: value bits resolved so far (key bits under kmask,
// inverted-position bits under pmask) and the rank still needed inside the
// current bin of in_bin entries.
struct SelState {
  uint32_t kpre, kmask, ppre, pmask, need, in_bin;
};

__device__ __forceinline__ bool in_prefix(const uint2 v, const SelState &s) {
  return (v.x & s.kmask) == s.kpre && ((kPosMask - v.y) & s.pmask) == s.ppre;
}

// Passes 2..5 of the select (key bits 10..20 and 0..9, then inverted
// position bits 8..18 and 0..7) over the entries the workgroup's threads hold
// (entry u of a thread present when bit u of `held` is set);
// done as soon as every entry of the current bin is taken.  The low-key-bit
// pass is skipped when every entry left after pass 2 shares those bits
// (seen during pass 2).  Once the key is resolved, up to kTieCap entries
// sharing it are ranked by position directly (the need-th lowest is the
// cut) instead of by the two position passes.  hist (kBins words) must be
// clear; it is clear again on return.  sh_word[0] / [1] / [5] must hold
// 0 / ~0 / 0 (or / and of low key bits, tie count); sh_word[2..4] and [6]
// carry results between threads; tie holds kTieCap positions.
__device__ __forceinline__ void late_passes(const uint2 (&ent)[kListChunks], uint32_t held,
                                            uint32_t *hist, uint32_t *scan, uint32_t *sh_word,
                                            uint32_t *tie, SelState &s) {
  const int tid = threadIdx.x, lane = tid % kWave;
  uint32_t lo_or = 0u, lo_and = ~0u;
#pragma unroll 1
  for (int pass = 1; pass < 5; ++pass) {
    if (s.need == s.in_bin) break;
    const bool on_pos = pass >= 3;
    const int shift = pass == 1 ? 10 : pass == 3 ? 8 : 0;
    const uint32_t dmask = pass == 2 ? 1023u : pass == 4 ? 255u : 2047u;
    if (pass == 3 && s.in_bin <= static_cast<uint32_t>(kTieCap)) {
      // the entries with the k-th key, by position: gather, rank, cut
#pragma unroll
      for (int u = 0; u < kListChunks; ++u) {
        const uint2 v = ent[u];
        if (((held >> u) & 1u) && v.x == s.kpre) tie[atomicAdd(&sh_word[5], 1u)] = v.y;
      }
      __syncthreads();
      if (tid < static_cast<int>(s.in_bin)) {
        const uint32_t mine = tie[tid];
        uint32_t below = 0;
#pragma unroll 1
        for (uint32_t j = 0; j < s.in_bin; ++j) below += tie[j] < mine;
        if (below + 1 == s.need) sh_word[6] = mine;
      }
      __syncthreads();
      s.ppre = kPosMask - sh_word[6];  // positions at or below the cut
      s.pmask = kPosMask;
      s.need = s.in_bin = 1u;
      break;
    }
    if (pass == 2) {
#pragma unroll
      for (int o = 32; o >= 1; o >>= 1) {
        lo_or |= __shfl_xor(lo_or, o, kWave);
        lo_and &= __shfl_xor(lo_and, o, kWave);
      }
      if (lane == 0) {
        atomicOr(&sh_word[0], lo_or);
        atomicAnd(&sh_word[1], lo_and);
      }
      __syncthreads();
      if (sh_word[0] == sh_word[1]) {
        // every entry left shares its low 10 key bits
        s.kpre |= sh_word[0];
        s.kmask |= 1023u;
        continue;
      }
    }
#pragma unroll
    for (int u = 0; u < kListChunks; ++u) {
      const uint2 v = ent[u];
      if (((held >> u) & 1u) && in_prefix(v, s)) {
        const uint32_t inv = kPosMask - v.y;
        atomicAdd(&hist[((on_pos ? inv : v.x) >> shift) & dmask], 1u);
        if (pass == 1) {
          // pooled over the sub-bins: a superset of the entries left
          lo_or |= v.x & 1023u;
          lo_and &= v.x & 1023u;
        }
      }
    }
    __syncthreads();
    find_digit<kSelThreads, 1>(hist, s.need, scan, &sh_word[2], &sh_word[3], &sh_word[4]);
    __syncthreads();
    const uint32_t digit = sh_word[2];
    if (on_pos) {
      s.ppre |= digit << shift;
      s.pmask |= dmask << shift;
    } else {
      s.kpre |= digit << shift;
      s.kmask |= dmask << shift;
    }
    s.need = sh_word[3];
    s.in_bin = sh_word[4];
    __syncthreads();  // sh_word[2..4] are rewritten by the next pass
  }
}

// Ascending write-out of the set marked in bits[0, ceil(c / 32)): sinks
// [0, lo) first, then the picked candidates, then the window [hi, c); the
// -1 tail.  Each thread writes its run of positions straight to the output
// (staging the set in LDS for coalesced stores cost a barrier and more).
__device__ void write_set(const uint32_t *bits, const Budget &bd, int n_sel, int32_t *dst,
                          uint32_t *scan) {
  const int tid = threadIdx.x;
  const int words = (bd.c + 31) / 32;
  const int per = (words + kSelThreads - 1) / kSelThreads;
  const int w0 = min(tid * per, words), w1 = min(w0 + per, words);
  uint32_t cnt = 0;
  for (int w = w0; w < w1; ++w) cnt += __popc(bits[w] & range_bits(32 * w, bd.lo, bd.hi));
  uint32_t n_picked;
  uint32_t out = bd.lo + block_exclusive_scan<kSelThreads>(cnt, scan, &n_picked);
  const int total = bd.lo + static_cast<int>(n_picked) + (bd.c - bd.hi);
  for (int j = tid; j < bd.lo && j < n_sel; j += kSelThreads) dst[j] = j;
  for (int j = tid; j < bd.c - bd.hi; j += kSelThreads) {
    const int at = bd.lo + static_cast<int>(n_picked) + j;
    if (at < n_sel) dst[at] = bd.hi + j;
  }
  for (int w = w0; w < w1; ++w) {
    uint32_t v = bits[w] & range_bits(32 * w, bd.lo, bd.hi);
    while (v) {
      const int j = __ffs(v) - 1;
      v &= v - 1;
      if (out < static_cast<uint32_t>(n_sel)) dst[out] = 32 * w + j;
      ++out;
    }
  }
  for (int s = total + tid; s < n_sel; s += kSelThreads) dst[s] = -1;
}

// ---------------------------------------------------------------------------
// Floors (one 1024-thread workgroup per row)
// ---------------------------------------------------------------------------
// The smallest score whose key is at or above `floor` (a key >= 2): a score
// f (not NaN) has key(f) >= floor exactly when f >= that score, and NaN
// (key 1) compares false.  Above every number's key: NaN (nothing passes).
__device__ __forceinline__ float floor_score(uint32_t floor) {
  if (floor >= 0x80000000u) return __uint_as_float(floor & 0x7fffffffu);  // +0 .. +inf, or NaN
  if (floor <= 0x007fffffu) return -__builtin_huge_valf();                // every number
  return __uint_as_float(~floor);                                         // -0 .. -max
}

// The two maps' shares of the budget, for the floors: the draft's m best,
// and the target's rest + m best (the draft's picks remove at most m).
__device__ __forceinline__ void floor_ranks(const Budget &bd, int kk[2]) {
  kk[0] = bd.m;
  kk[1] = min(bd.rest + bd.m, bd.hi - bd.lo);
}

struct FloorShared {
  uint32_t hist[2][kBins];          // sample histograms of the two maps
  uint32_t scan[kSelWaves];
  uint32_t digit[2], need[2], digit_hi[2];
};

// Per row and map, the floor key: the 22-bit prefix of the r-th largest
// in-range sample key (r a few standard deviations above the rank the k-th
// best candidate would have in the sample), or 1 (every candidate) when the
// sample is too small for r or the map has no share.  With it a shift s:
// the top of the 11-bit bin of the r'-th largest sample key (r' as many
// deviations below that rank) is an upper estimate U of the k-th best, and
// (U - floor) >> s < 1024, so floor-relative bins (key - floor) >> s split
// [floor, U] into at most 1024 bins.  floors[row][map] = {floor, s}.
__global__ __launch_bounds__(kSelThreads) void select_floor_kernel(
    const float *draft, const float *target, int score_len, const int32_t *ctx_lens, int hkv,
    int n_sel, int n_sink, int n_recent, int n_draft_top, uint32_t *floors) {
  __shared__ FloorShared sh;
  const int tid = threadIdx.x;
  const int bg = blockIdx.x;
  const int64_t row0 = static_cast<int64_t>(bg) * score_len;
  // the sample, entry tid + 1024 u, loaded before the context length is
  // known (positions outside the candidates are not used)
  const int n_smp = min(score_len, kSample);
  uint32_t raw[2][kSmpPer];
#pragma unroll
  for (int u = 0; u < kSmpPer; ++u) {
    const int p = sample_pos(min(tid + kSelThreads * u, n_smp - 1), score_len);
    raw[0][u] = __float_as_uint(draft[row0 + p]);
    raw[1][u] = __float_as_uint(target[row0 + p]);
  }
  const Budget bd = budget(ctx_lens[bg / hkv], score_len, n_sel, n_sink, n_recent, n_draft_top);
  const int n_cand = bd.hi - bd.lo;
  int kk[2];
  floor_ranks(bd, kk);
  uint32_t key[2][kSmpPer];
#pragma unroll
  for (int u = 0; u < kSmpPer; ++u) {
    const int i = tid + kSelThreads * u;
    const int p = sample_pos(min(i, n_smp - 1), score_len);
    const bool in = i < n_smp && p >= bd.lo && p < bd.hi;
#pragma unroll
    for (int map = 0; map < 2; ++map)
      key[map][u] = in ? order_key(__uint_as_float(raw[map][u])) : 0u;
  }
  const int n_in = sample_in_range(bd.lo, bd.hi, score_len);
  bool use[2];
  uint32_t need[2], need_hi[2];
#pragma unroll
  for (int map = 0; map < 2; ++map) {
    const float mean = kk[map] > 0 ? static_cast<float>(kk[map]) * n_in / n_cand : 0.f;
    need[map] = static_cast<uint32_t>(ceilf(mean + 3.f * sqrtf(mean) + 8.f));
    need_hi[map] = static_cast<uint32_t>(fmaxf(1.f, floorf(mean - 3.f * sqrtf(mean) - 8.f)));
    use[map] = kk[map] > 0 && need[map] < static_cast<uint32_t>(n_in);
  }
  for (int i = tid; i < 2 * kBins; i += kSelThreads) (&sh.hist[0][0])[i] = 0u;
  __syncthreads();
  uint32_t prefix[2] = {0u, 0u}, pmask = 0u;
  if (use[0] || use[1]) {
#pragma unroll 1
    for (int pass = 0; pass < 2; ++pass) {
      const int shift = pass == 0 ? 21 : 10;
#pragma unroll
      for (int u = 0; u < kSmpPer; ++u)
#pragma unroll
        for (int map = 0; map < 2; ++map)
          if (use[map] && key[map][u] != 0u && (key[map][u] & pmask) == prefix[map])
            atomicAdd(&sh.hist[map][(key[map][u] >> shift) & (kBins - 1)], 1u);
      __syncthreads();
      // both maps' digit searches share one scan: counts of at most kSample
      // each, packed in the low and high 16 bits
      {
        constexpr int kPer = kBins / kSelThreads;
        const int top = kBins - 1 - kPer * tid;
        uint32_t cnt[2][kPer], mine = 0;
#pragma unroll
        for (int map = 0; map < 2; ++map)
#pragma unroll
          for (int i = 0; i < kPer; ++i) {
            cnt[map][i] = sh.hist[map][top - i];
            sh.hist[map][top - i] = 0u;
            mine += cnt[map][i] << (16 * map);
          }
        uint32_t all;
        const uint32_t above2 = block_exclusive_scan<kSelThreads, false>(mine, sh.scan, &all);
#pragma unroll
        for (int map = 0; map < 2; ++map) {
          uint32_t above = (above2 >> (16 * map)) & 0xffffu;
#pragma unroll
          for (int i = 0; i < kPer; ++i) {
            if (above < need[map] && need[map] <= above + cnt[map][i]) {
              sh.digit[map] = static_cast<uint32_t>(top - i);
              sh.need[map] = need[map] - above;
            }
            if (pass == 0 && above < need_hi[map] && need_hi[map] <= above + cnt[map][i])
              sh.digit_hi[map] = static_cast<uint32_t>(top - i);
            above += cnt[map][i];
          }
        }
      }
      __syncthreads();
#pragma unroll
      for (int map = 0; map < 2; ++map) {
        prefix[map] |= sh.digit[map] << shift;
        need[map] = sh.need[map];
      }
      pmask |= static_cast<uint32_t>(kBins - 1) << shift;
      __syncthreads();  // sh.digit / sh.need are rewritten by the next pass
    }
  }
  if (tid < 2) {
    const int map = tid;
    uint32_t floor = 1u, sft = 21u;  // no floor: bins of the top 11 key bits
    if (use[map]) {
      floor = max(prefix[map], 1u);
      const uint32_t dh = sh.digit_hi[map];
      const uint32_t upper = dh >= kBins - 1 ? ~0u : ((dh + 1u) << 21) - 1u;
      const uint32_t span = upper - floor;  // the r'-th key is at or above the r-th
      sft = static_cast<uint32_t>(max(0, (31 - __builtin_clz(span | 1u)) - 9));
    }
    floors[4 * bg + 2 * map] = floor;
    floors[4 * bg + 2 * map + 1] = sft;
  }
}

// ---------------------------------------------------------------------------
// Filter (one 256-thread workgroup per 8192-position chunk, both maps)
// ---------------------------------------------------------------------------
struct FiltShared {
  uint4 stage[kChunk / 4];          // one map's chunk scores
  uint32_t n_out[2];                // list entries of the chunk
};

__global__ __launch_bounds__(kFiltThreads) void select_filter_kernel(
    const float *draft, const float *target, int score_len, const int32_t *ctx_lens, int hkv,
    int n_sel, int n_sink, int n_recent, int n_draft_top, int nch, const uint32_t *floors,
    uint32_t *counts, uint2 *lists) {
  __shared__ FiltShared sh;
  const int tid = threadIdx.x, lane = tid % kWave;
  // Chunk-major block order: block i goes to XCD i mod 8, so with a multiple
  // of 8 rows all chunks of row bg run on the XCD of bg mod 8, where the
  // floor and list kernels' workgroup for that row runs too (their data
  // stays in that XCD's L2).
  const int rows_n = gridDim.x / nch;
  const int bg = blockIdx.x % rows_n, ch = blockIdx.x / rows_n;
  const int64_t row0 = static_cast<int64_t>(bg) * score_len;
  const float *rows[2] = {draft + row0, target + row0};
  const int c0 = ch * kChunk;

  // The chunk (positions c0 + 4*(tid + 256 u) + e), one 16-byte load per
  // map and u through buffer resources that end at the row's end (dword
  // alignment suffices), issued before the context length is known;
  // positions outside the candidates are loaded but not used.  A load that
  // would pass the row's end is moved back to end there and its values are
  // not used; the partial quad at the end is read with single loads.  Every
  // load is unconditional: the compiler waits at once for a conditional one.
  const __amdgpu_buffer_rsrc_t rs[2] = {
      __builtin_amdgcn_make_buffer_rsrc(const_cast<float *>(rows[0]), 0, score_len * 4,
                                        kBufferFlags),
      __builtin_amdgcn_make_buffer_rsrc(const_cast<float *>(rows[1]), 0, score_len * 4,
                                        kBufferFlags)};
  uint32_t x[2][kQuads][4];
#pragma unroll
  for (int u = 0; u < kQuads; ++u) {
    const int p4 = c0 + 4 * (tid + kFiltThreads * u);
    const int off = max(min(p4, score_len - 4), 0) * 4;
#pragma unroll
    for (int map = 0; map < 2; ++map) {
      const auto q = __builtin_amdgcn_raw_buffer_load_b128(rs[map], off, 0, 0);
      x[map][u][0] = q[0], x[map][u][1] = q[1], x[map][u][2] = q[2], x[map][u][3] = q[3];
    }
  }
  const int ep = (score_len & ~3) + tid;  // threads 0..3: the partial quad at the end
  uint32_t ex[2];
#pragma unroll
  for (int map = 0; map < 2; ++map)
    ex[map] = __builtin_amdgcn_raw_buffer_load_b32(rs[map], (tid < 4 ? ep : 0) * 4, 0, 0);

  const Budget bd = budget(ctx_lens[bg / hkv], score_len, n_sel, n_sink, n_recent, n_draft_top);
  const int p_begin = max(c0, bd.lo), p_end = min(c0 + kChunk, bd.hi);
  int kk[2];
  floor_ranks(bd, kk);
  bool want[2];
#pragma unroll
  for (int map = 0; map < 2; ++map) want[map] = kk[map] > 0 && p_end > p_begin;
  uint32_t *count = counts + (static_cast<int64_t>(bg) * nch + ch) * 2;
  if (!want[0] && !want[1]) {
    if (tid < 2) count[tid] = 0;
    return;
  }
  const bool ev = tid < 4 && ep < score_len && ep >= p_begin && ep < p_end;
  if (tid < 2) sh.n_out[tid] = 0u;

  // the floors as scores: a score passes when it compares >= fl (all:
  // floor 1, every candidate, NaN included)
  float fl[2];
  bool all[2];
#pragma unroll
  for (int map = 0; map < 2; ++map) {
    const uint32_t floor = floors[4 * bg + 2 * map];
    all[map] = floor <= 1u;
    fl[map] = floor_score(max(floor, 2u));
  }
  // per map, this thread's passing scores as a 32-bit mask (bit 4u + e)
  const bool inside = c0 >= bd.lo && c0 + kChunk <= bd.hi;  // every quad whole and a candidate
  uint32_t mask[2] = {0u, 0u};
#pragma unroll
  for (int map = 0; map < 2; ++map) {
    if (!want[map]) continue;
#pragma unroll
    for (int u = 0; u < kQuads; ++u) {
      const int p4 = c0 + 4 * (tid + kFiltThreads * u);
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const float f = __uint_as_float(x[map][u][e]);
        bool pass = all[map] || f >= fl[map];
        if (!inside) pass = pass && p4 + 3 < score_len && p4 + e >= p_begin && p4 + e < p_end;
        mask[map] |= pass ? 1u << (4 * u + e) : 0u;
      }
    }
  }
  bool epass[2];
#pragma unroll
  for (int map = 0; map < 2; ++map)
    epass[map] = want[map] && ev && (all[map] || __uint_as_float(ex[map]) >= fl[map]);
  __syncthreads();  // sh.n_out is clear
  // this wave's slots, reserved with one LDS atomic per map
  uint32_t slot[2];
#pragma unroll
  for (int map = 0; map < 2; ++map) {
    const uint32_t n = static_cast<uint32_t>(__popc(mask[map])) + (epass[map] ? 1u : 0u);
    const uint32_t incl = wave_inclusive_scan(n);
    uint32_t base = 0;
    if (lane == kWave - 1 && incl != 0u) base = atomicAdd(&sh.n_out[map], incl);
    slot[map] = __shfl(base, kWave - 1, kWave) + incl - n;
  }
  // per map: its chunk scores into LDS, then each thread appends its
  // passing ones from there (raw score bits and position)
#pragma unroll
  for (int map = 0; map < 2; ++map) {
    if (!want[map]) continue;
    __syncthreads();  // the stage is free
#pragma unroll
    for (int u = 0; u < kQuads; ++u)
      sh.stage[tid + kFiltThreads * u] =
          make_uint4(x[map][u][0], x[map][u][1], x[map][u][2], x[map][u][3]);
    __syncthreads();
    uint2 *list = lists + ((static_cast<int64_t>(bg) * nch + ch) * 2 + map) * kChunkCap;
    const uint32_t *st = reinterpret_cast<const uint32_t *>(&sh.stage[0]);
    uint32_t m = mask[map], sl = slot[map];
    while (m) {
      const int i = __ffs(m) - 1;
      m &= m - 1;
      const int q = tid + kFiltThreads * (i >> 2);
      if (sl < static_cast<uint32_t>(kChunkCap))
        list[sl] = make_uint2(st[4 * q + (i & 3)], c0 + 4 * q + (i & 3));
      ++sl;
    }
    if (epass[map] && sl < static_cast<uint32_t>(kChunkCap)) list[sl] = make_uint2(ex[map], ep);
  }
  __syncthreads();
  if (tid < 2) count[tid] = want[tid] ? sh.n_out[tid] : 0u;
}

// ---------------------------------------------------------------------------
// Per-row select over the lists
// ---------------------------------------------------------------------------
struct alignas(16) SelBufs {
  uint32_t hist_first[kBins * kCopies];  // the first digit
  uint32_t hist1[kBins];            // later passes
  uint32_t tie[kTieCap];            // positions of the entries with the k-th key
  uint2 cand[kRankCap];             // entries of the k-th value's floor-relative bin
};
struct alignas(16) ListShared {
  uint32_t bits[kWords];            // chosen positions of the row
  uint32_t hist_t[kBins * kCopies]; // the target map's first histogram
  uint2 stash[kListChunks][kSelThreads];  // the target's entries while the draft's run
  union {
    SelBufs s;
    StreamShared stream;            // the fallback
  };
  uint32_t scan[kSelWaves];
  uint32_t word[8];                 // small results passed between threads
};

// Floor-relative bin of a listed key (every listed key is at or above the
// floor): (key - floor) >> sft, the keys past the upper estimate in the last
// bin.
__device__ __forceinline__ uint32_t rel_bin(uint32_t key, uint32_t floor, uint32_t sft) {
  return min((key - floor) >> sft, static_cast<uint32_t>(kBins - 1));
}

// Value order of two listed entries: key, then the lower position.
__device__ __forceinline__ bool value_above(const uint2 a, const uint2 b) {
  return a.x > b.x || (a.x == b.x && a.y < b.y);
}

// The exact k best (k >= 1) of the listed entries into `bits`: entry u of a
// thread (key, position) is listed when bit u of `held` is set, and `first`
// holds the listed entries' floor-relative bin counts; false (nothing
// marked) if fewer than k are listed.  When the k-th value's bin holds at
// most kRankCap entries, those are ranked directly; otherwise the bins are
// rebuilt from the top 11 key bits and the radix passes resolve the rest.
// `first`, hist_first and hist1 are clear on return.
__device__ __forceinline__ bool list_select(const uint2 (&ent)[kListChunks], uint32_t held,
                                            uint32_t k, ListShared &sh, uint32_t *first,
                                            uint32_t floor, uint32_t sft) {
  const int tid = threadIdx.x, lane = tid % kWave;
  SelBufs &B = sh.s;
  if (tid == 0) {
    sh.word[0] = 0u;   // or of low key bits
    sh.word[1] = ~0u;  // and
    sh.word[5] = 0u;   // entries gathered (bin, then ties)
  }
  const uint32_t total =
      find_digit<kSelThreads, kCopies>(first, k, sh.scan, &sh.word[2], &sh.word[3], &sh.word[4]);
  __syncthreads();
  if (total < k) return false;
  SelState s;
  s.need = sh.word[3];
  s.in_bin = sh.word[4];
  const uint32_t d1 = sh.word[2];
  __syncthreads();  // sh.word[2..4] are rewritten below
  if (s.in_bin <= static_cast<uint32_t>(kRankCap)) {
    // the bin's entries, ranked by value: the need-th is the k-th overall
#pragma unroll
    for (int u = 0; u < kListChunks; ++u) {
      const uint2 v = ent[u];
      if (((held >> u) & 1u) && rel_bin(v.x, floor, sft) == d1)
        B.cand[atomicAdd(&sh.word[5], 1u)] = v;
    }
    __syncthreads();
    if (tid < static_cast<int>(s.in_bin)) {
      const uint2 mine = B.cand[tid];
      uint32_t above = 0;
#pragma unroll 1
      for (uint32_t j = 0; j < s.in_bin; ++j) above += value_above(B.cand[j], mine);
      if (above + 1 == s.need) {
        sh.word[2] = mine.x;
        sh.word[3] = mine.y;
      }
    }
    __syncthreads();
    s.kpre = sh.word[2];
    s.kmask = ~0u;
    s.ppre = kPosMask - sh.word[3];  // positions at or below the k-th's
    s.pmask = kPosMask;
  } else {
    // bins of the top 11 key bits (hist_first is clear: it was never used,
    // or it was `first` and the search read it all)
    const uint32_t copy = static_cast<uint32_t>(lane) & (kCopies - 1);
#pragma unroll
    for (int u = 0; u < kListChunks; ++u)
      if ((held >> u) & 1u) atomicAdd(&B.hist_first[hslot<kCopies>(ent[u].x >> 21, copy)], 1u);
    if (tid == 0) sh.word[5] = 0u;
    __syncthreads();
    find_digit<kSelThreads, kCopies>(B.hist_first, k, sh.scan, &sh.word[2], &sh.word[3], &sh.word[4]);
    __syncthreads();
    s.kpre = sh.word[2] << 21;
    s.kmask = static_cast<uint32_t>(kBins - 1) << 21;
    s.ppre = s.pmask = 0u;
    s.need = sh.word[3];
    s.in_bin = sh.word[4];
    __syncthreads();  // sh.word[2..4] are rewritten below
    late_passes(ent, held, B.hist1, sh.scan, sh.word, B.tie, s);
  }
  // every value at or above the k-th: above its bin in the resolved key
  // bits, or inside it and at or above it in the resolved position bits
#pragma unroll
  for (int u = 0; u < kListChunks; ++u) {
    const uint2 v = ent[u];
    const uint32_t kx = v.x & s.kmask;
    if (((held >> u) & 1u) &&
        (kx > s.kpre || (kx == s.kpre && ((kPosMask - v.y) & s.pmask) >= s.ppre)))
      atomicOr(&sh.bits[v.y >> 5], 1u << (v.y & 31));
  }
  __syncthreads();
  return true;
}

__global__ __launch_bounds__(kSelThreads) void select_lists_kernel(
    const float *draft, const float *target, int score_len, const int32_t *ctx_lens, int hkv,
    int n_sel, int n_sink, int n_recent, int n_draft_top, int nch, const uint32_t *floors,
    const uint32_t *counts, const uint2 *lists, int32_t *kv_idx) {
  __shared__ ListShared sh;
  const int tid = threadIdx.x, lane = tid % kWave;
  const int bg = blockIdx.x;

  // Every list slot this thread holds (raw score bits and position) is
  // loaded before anything waits: slot (tid + 128 u) mod 1024 of chunk u of
  // both maps.  A chunk's list fills its first slots, so the rotation gives
  // every thread a share of the entries rather than all eight slots to the
  // first few hundred threads.  Chunks past nch repeat the last one and are
  // dropped below.
  constexpr int kTurn = kChunkCap / kListChunks;
  static_assert(kSelThreads == kChunkCap, "one slot of each chunk per thread");
  uint2 e[2][kListChunks];
  {
    const uint2 *src = lists + static_cast<int64_t>(bg) * nch * 2 * kChunkCap;
#pragma unroll
    for (int u = 0; u < kListChunks; ++u)
#pragma unroll
      for (int map = 0; map < 2; ++map)
        e[map][u] = src[(static_cast<int64_t>(min(u, nch - 1)) * 2 + map) * kChunkCap +
                        ((tid + kTurn * u) & (kChunkCap - 1))];
  }
  const Budget bd = budget(ctx_lens[bg / hkv], score_len, n_sel, n_sink, n_recent, n_draft_top);
  const int words = (bd.c + 31) / 32;
  for (int w = tid; w < words; w += kSelThreads)
    sh.bits[w] = range_bits(32 * w, 0, bd.lo) | range_bits(32 * w, bd.hi, bd.c);
  // a slot holds an entry below its chunk's count; a count past the slots
  // means the chunk's list overflowed, and so does any entry in a chunk
  // past the first kListChunks (no slots here for it)
  bool over[2] = {false, false};
  uint32_t valid[2] = {0u, 0u};
#pragma unroll
  for (int u = 0; u < kListChunks; ++u)
#pragma unroll
    for (int map = 0; map < 2; ++map) {
      const uint32_t n = u < nch ? counts[(static_cast<int64_t>(bg) * nch + u) * 2 + map] : 0u;
      over[map] = over[map] || n > static_cast<uint32_t>(kChunkCap);
      if (static_cast<uint32_t>((tid + kTurn * u) & (kChunkCap - 1)) < n) valid[map] |= 1u << u;
    }
  for (int u = kListChunks; u < nch; ++u)
#pragma unroll
    for (int map = 0; map < 2; ++map)
      over[map] = over[map] || counts[(static_cast<int64_t>(bg) * nch + u) * 2 + map] != 0u;
  for (int i = tid; i < kBins * (kCopies + 1); i += kSelThreads) sh.s.hist_first[i] = 0u;
  for (int i = tid; i < kBins * kCopies; i += kSelThreads) sh.hist_t[i] = 0u;
  __syncthreads();

  // Both maps' entries stay in registers.  One pass turns their scores into
  // keys and counts them into the maps' first histograms (floor-relative
  // bins); the target's still counts the entries the draft will pick, which
  // leave it once they are known.
  uint32_t fl[2], sf[2];
  bool use[2];
  const uint32_t copy = static_cast<uint32_t>(lane) & (kCopies - 1);
#pragma unroll
  for (int map = 0; map < 2; ++map) {
    fl[map] = floors[4 * bg + 2 * map];
    sf[map] = floors[4 * bg + 2 * map + 1];
    use[map] = (map == 0 ? bd.m : bd.rest) > 0 && !over[map];
    if (!use[map]) continue;
    uint32_t *first = map == 0 ? sh.s.hist_first : sh.hist_t;
    uint32_t n_top = 0;  // entries past the upper estimate: counted per wave
#pragma unroll
    for (int u = 0; u < kListChunks; ++u) {
      if (!((valid[map] >> u) & 1u)) continue;
      const uint32_t key = order_key(__uint_as_float(e[map][u].x));
      e[map][u].x = key;
      const uint32_t bin = rel_bin(key, fl[map], sf[map]);
      if (bin == kBins - 1)
        ++n_top;
      else
        atomicAdd(&first[hslot<kCopies>(bin, copy)], 1u);
    }
    n_top = wave_inclusive_scan(n_top);
    if (lane == kWave - 1 && n_top != 0u) atomicAdd(&first[hslot<kCopies>(kBins - 1, 0)], n_top);
  }
  // the target's entries wait in this thread's LDS slots, so that one set
  // of registers holds the current map's
  if (use[1]) {
#pragma unroll
    for (int u = 0; u < kListChunks; ++u) sh.stash[u][tid] = e[1][u];
  }
  __syncthreads();

  // The draft's m best, then the target's rest best among the candidates
  // the draft left: each over its list, or by the streaming fallback.  One
  // code path serves both maps.
  const int64_t row0 = static_cast<int64_t>(bg) * score_len;
  uint2 ent[kListChunks];
#pragma unroll
  for (int u = 0; u < kListChunks; ++u) ent[u] = e[0][u];
#pragma unroll 1
  for (int map = 0; map < 2; ++map) {
    const int k = map == 0 ? bd.m : bd.rest;
    if (k <= 0) continue;
    uint32_t held = map == 0 ? valid[0] : valid[1];
    const bool use_list = map == 0 ? use[0] : use[1];
    if (map == 1) {
      if (use_list) {
#pragma unroll
        for (int u = 0; u < kListChunks; ++u) {
          ent[u] = sh.stash[u][tid];
          const bool ok = (held >> u) & 1u;
          const uint32_t py = ok ? ent[u].y : 0u;  // an empty slot's position is not read
          if (ok && ((sh.bits[py >> 5] >> (py & 31)) & 1u)) {
            held &= ~(1u << u);
            atomicSub(&sh.hist_t[hslot<kCopies>(rel_bin(ent[u].x, fl[1], sf[1]), copy)], 1u);
          }
        }
      }
      // the draft's streaming fallback shares these buffers
      for (int i = tid; i < kBins * (kCopies + 1); i += kSelThreads) sh.s.hist_first[i] = 0u;
      __syncthreads();
    }
    bool done = false;
    if (use_list)
      done = list_select(ent, held, static_cast<uint32_t>(k), sh,
                         map == 0 ? sh.s.hist_first : sh.hist_t, map == 0 ? fl[0] : fl[1],
                         map == 0 ? sf[0] : sf[1]);
    if (!done)
      select_best((map == 0 ? draft : target) + row0, bd.lo, bd.hi, static_cast<uint32_t>(k),
                  sh.bits, sh.stream);
  }
  write_set(sh.bits, bd, n_sel, kv_idx + static_cast<int64_t>(bg) * n_sel, sh.scan);
}

// ---------------------------------------------------------------------------
// Longer rows: the streaming select for both maps
// ---------------------------------------------------------------------------
struct StreamKernelShared {
  StreamShared stream;
  uint32_t scan[kSelWaves];
};

__global__ __launch_bounds__(kSelThreads) void select_stream_kernel(
    const float *draft, const float *target, int score_len, const int32_t *ctx_lens, int hkv,
    int n_sel, int n_sink, int n_recent, int n_draft_top, int32_t *kv_idx) {
  extern __shared__ uint32_t bits[];  // ceil(score_len / 32) words
  __shared__ StreamKernelShared sh;
  const int tid = threadIdx.x;
  const int bg = blockIdx.x;
  const Budget bd = budget(ctx_lens[bg / hkv], score_len, n_sel, n_sink, n_recent, n_draft_top);
  const int words = (bd.c + 31) / 32;
  for (int w = tid; w < words; w += kSelThreads)
    bits[w] = range_bits(32 * w, 0, bd.lo) | range_bits(32 * w, bd.hi, bd.c);
  __syncthreads();
  const int64_t row0 = static_cast<int64_t>(bg) * score_len;
  if (bd.m > 0) select_best(draft + row0, bd.lo, bd.hi, static_cast<uint32_t>(bd.m), bits, sh.stream);
  if (bd.rest > 0)
    select_best(target + row0, bd.lo, bd.hi, static_cast<uint32_t>(bd.rest), bits, sh.stream);
  write_set(bits, bd, n_sel, kv_idx + static_cast<int64_t>(bg) * n_sel, sh.scan);
}

}  // namespace

int select_max_positions() { return 1 << kPosBits; }

namespace {
int select_chunks(int score_len) { return (score_len + kChunk - 1) / kChunk; }
size_t select_count_bytes(size_t rows, int nch) {
  return (rows * static_cast<size_t>(nch) * 2 * sizeof(uint32_t) + 255) / 256 * 256;
}
size_t select_floor_bytes(size_t rows) { return (rows * 4 * sizeof(uint32_t) + 255) / 256 * 256; }
}  // namespace

size_t select_workspace_bytes(int batch, int hkv, int score_len) {
  if (score_len > kBitsMax) return 256;  // the streaming kernel needs none
  const size_t rows = static_cast<size_t>(batch) * hkv;
  const int nch = select_chunks(score_len);
  return select_floor_bytes(rows) + select_count_bytes(rows, nch) +
         rows * static_cast<size_t>(nch) * 2 * kChunkCap * sizeof(uint2);
}

hipError_t launch_select_kv_idx(const float *draft, const float *target, int score_len,
                                const int32_t *ctx_lens, int batch, int hkv, int n_sel,
                                int n_sink, int n_recent, int n_draft_top, int32_t *kv_idx,
                                void *workspace, hipStream_t s) {
  if (score_len < 1 || score_len > select_max_positions()) return hipErrorInvalidValue;
  const size_t rows = static_cast<size_t>(batch) * hkv;
  if (score_len > kBitsMax) {
    const size_t lds = static_cast<size_t>((score_len + 31) / 32) * sizeof(uint32_t);
    hipLaunchKernelGGL(select_stream_kernel, dim3(static_cast<unsigned>(rows)), dim3(kSelThreads),
                       lds, s, draft, target, score_len, ctx_lens, hkv, n_sel, n_sink, n_recent,
                       n_draft_top, kv_idx);
    return hipGetLastError();
  }
  const int nch = select_chunks(score_len);
  char *ws = static_cast<char *>(workspace);
  uint32_t *floors = reinterpret_cast<uint32_t *>(ws);
  uint32_t *counts = reinterpret_cast<uint32_t *>(ws + select_floor_bytes(rows));
  uint2 *lists = reinterpret_cast<uint2 *>(ws + select_floor_bytes(rows) +
                                           select_count_bytes(rows, nch));
  hipLaunchKernelGGL(select_floor_kernel, dim3(static_cast<unsigned>(rows)), dim3(kSelThreads), 0,
                     s, draft, target, score_len, ctx_lens, hkv, n_sel, n_sink, n_recent,
                     n_draft_top, floors);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(select_filter_kernel, dim3(static_cast<unsigned>(rows * nch)),
                     dim3(kFiltThreads), 0, s, draft, target, score_len, ctx_lens, hkv, n_sel,
                     n_sink, n_recent, n_draft_top, nch, floors, counts, lists);
  e = hipGetLastError();
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(select_lists_kernel, dim3(static_cast<unsigned>(rows)), dim3(kSelThreads), 0,
                     s, draft, target, score_len, ctx_lens, hkv, n_sel, n_sink, n_recent,
                     n_draft_top, nch, floors, counts, lists, kv_idx);
  return hipGetLastError();
}

}  // namespace hsv
