// Partial verification attention for small query groups on gfx950: at most
// 32 grouped rows per KV head (e.g. 4 query heads x an 8-token draft block),
// bf16, D = 128.  The key set is one range: the dense prefix [0, c) or the
// gathered index set (Dustin page, verification over the selected subset of
// a fully indexed cache), followed by the N draft rows.
//
// With 32 query rows every K/V byte feeds only 32 x 128 x 2 multiply-adds,
// so the kernel is an HBM stream and its job is to keep enough bytes in
// flight.  One workgroup owns one (split, sequence, KV head); its W waves
// (two for dense calls, four for sparse ones: Cfg below) take every W-th
// 32-key block of the split, each with its own online softmax, and merge
// their results through LDS at the end.  Each wave moves its blocks
// HBM -> LDS with global_load_lds_dwordx4 into a private two-stage ring and
// waits only on its own DMA (s_waitcnt vmcnt), so the loop has no workgroup
// barrier and the streams drift freely.  A dense workgroup takes 66.5 KB of
// LDS, so two run on each CU (one wave per SIMD): while one starts (query
// loads, first DMA) or ends (merge, partial stores), the other keeps
// streaming.
//
// Inside a block everything is as in the 256-row kernel (attn_dma.hip): the
// 1 KB DMA blocks (K: (chunk%4)*256 + (key%16)*16, V: (key%16)*64 +
// (chunk%4)*16), S^T = K.Q^T and O^T += V^T.P^T on v_mfma_f32_32x32x16_bf16
// with one lane per query column, V^T by ds_read_b64_tr_b16, the log2-domain
// softmax with a fast path and exact fp32 row sums, and the unified key range
// [0, c+N) whose rows at or past c are masked by the ancestor bits.  The
// split's result is written as a scaled-fp16 partial row (see attn_dma.hip).
//
// Sparse sets: key t < n_sel is cache row kv_idx[t], key n_sel + j is draft
// row c + j.  Every DMA lane supplies its own address, so gathering costs
// nothing extra on the data path; the row numbers of a block are themselves
// fetched by a 4-byte-per-lane DMA into a per-wave two-slot LDS ring two
// blocks ahead, so no load the compiler tracks ever sits between the DMA
// waits.  Indices outside [0, c) are masked (a per-block 32-bit validity
// word taken by ballot when the block's rows are read).
//
// Sparse sets over a paged cache: the sequence's block table is copied into
// LDS once, and every gathered row (index or draft row) goes through it to a
// 64-bit pool address per lane, so the pool may be of any size.
#include "common.hpp"
#include "launch.h"

namespace hsv {
namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef float floatx16 __attribute__((ext_vector_type(16)));
typedef float floatx8 __attribute__((ext_vector_type(8)));
typedef float floatx4 __attribute__((ext_vector_type(4)));
typedef _Float16 halfx8 __attribute__((ext_vector_type(8)));
typedef __attribute__((address_space(3))) char lds_char;
typedef __attribute__((address_space(3))) bf16x4 lds_bf16x4;
typedef __attribute__((address_space(3))) bf16x8 lds_bf16x8;
typedef __attribute__((address_space(3))) int32_t lds_i32;

constexpr int kRows = 32;                     // grouped query rows (one MFMA column block)
constexpr int kBK = 32;                       // keys per block
constexpr int kD = 128;
constexpr int kRowBytes = kD * 2;
constexpr int kHalfBytes = kBK * kRowBytes;   // K (or V) of one block: 8 KB
constexpr int kBlockBytes = 2 * kHalfBytes;   // 16 KB
constexpr int kRing = 2;                      // stages per wave
constexpr int kWaveLds = kRing * kBlockBytes; // 32 KB
constexpr int kDmaPerBlock = 2 * kHalfBytes / 1024;  // 16 one-KB DMA instructions
// Epilogue: each wave's 32 x 128 fp32 accumulator rows (padded) and row stats.
constexpr int kEpiRow = kD * 4 + 16;
constexpr int kIdxSlot = 64 * 4;               // one block's row indices (64 lanes)

// Workgroup shape.  Dense calls run two waves per workgroup and two
// workgroups per CU, so one workgroup's start and end hide behind the
// other's stream (ragged batches run several rounds of workgroups).  Sparse
// calls (index sets of one length, usually a single round) run four waves
// and one workgroup per CU: fewer workgroups, epilogues and partials.
template <int W>
struct Cfg {
  static constexpr int kWaves = W;             // waves per workgroup, each on its own blocks
  static constexpr int kNT = W * 64;
  static constexpr int kWgPerCu = W == 2 ? 2 : 1;
  static constexpr int kEpiBytes = W * kRows * kEpiRow + 2 * W * kRows * 4;
  // the final combination: kEpiTpr threads per row, kEpiFeat features each
  static constexpr int kEpiTpr = kNT / kRows;
  static constexpr int kEpiFeat = kD / kEpiTpr;
  static constexpr int kStreamBytes = W * kWaveLds;
  static constexpr int kIdxBytes = W * 2 * kIdxSlot;
  static constexpr int kSmemBytes =
      (kStreamBytes > kEpiBytes ? kStreamBytes : kEpiBytes) + kIdxBytes;
  static_assert(kEpiTpr * kEpiFeat == kD && (kEpiTpr & (kEpiTpr - 1)) == 0, "epilogue split");
  static_assert(kWgPerCu * kSmemBytes <= 160 * 1024, "LDS of the CU's workgroups");
};
constexpr int waves_for(bool sparse) { return sparse ? 4 : 2; }
// sparse over a paged cache: the sequence's block table, after the rest
constexpr int kTabEntries = 6144;
constexpr int kTabBytes = kTabEntries * 4;
static_assert(Cfg<waves_for(true)>::kSmemBytes + kTabBytes <= 160 * 1024, "LDS of one workgroup");

constexpr float kSumLimit = 65536.f;  // as in attn_dma.hip

// (M0 is clobbered on purpose: nothing else in these kernels uses it.)
#pragma clang diagnostic push
#pragma clang diagnostic ignored "-Winline-asm"
__device__ __forceinline__ void dma16(const char *sbase, uint32_t voff, uint32_t lds_base) {
  asm volatile(
      "s_mov_b32 m0, %2\n\t"
      "s_nop 0\n\t"
      "global_load_lds_dwordx4 %0, %1"
      :
      : "v"(voff), "s"(sbase), "s"(lds_base)
      : "memory", "m0");
}

// The same with a 64-bit address per lane (gathers from a paged pool).
__device__ __forceinline__ void dma16p(const char *addr, uint32_t lds_base) {
  asm volatile(
      "s_mov_b32 m0, %1\n\t"
      "s_nop 0\n\t"
      "global_load_lds_dwordx4 %0, off"
      :
      : "v"(addr), "s"(lds_base)
      : "memory", "m0");
}

// Row indices of one block (64 lanes x 4 bytes; lanes 32..63 repeat 0..31).
__device__ __forceinline__ void dma4(const char *sbase, uint32_t voff, uint32_t lds_base) {
  asm volatile(
      "s_mov_b32 m0, %2\n\t"
      "s_nop 0\n\t"
      "global_load_lds_dword %0, %1"
      :
      : "v"(voff), "s"(sbase), "s"(lds_base)
      : "memory", "m0");
}
#pragma clang diagnostic pop

// s_waitcnt vmcnt(n) for the counts this kernel uses: 0, 16 (one block's 16
// DMA instructions still in flight) and 17 (a block and one index fetch).
__device__ __forceinline__ void wait_vm(int n) {
  static_assert(kDmaPerBlock == 16, "the immediates below");
  if (n >= 17)
    asm volatile("s_waitcnt vmcnt(17)" ::: "memory");
  else if (n >= 16)
    asm volatile("s_waitcnt vmcnt(16)" ::: "memory");
  else
    asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
}

// ---- slots of a ragged dense batch ---------------------------------------------
// With equal slot counts the workgroups of a long sequence run longer than
// those of a short one, and the batch ends on a few long workgroups.  Here
// sequence b instead gets n_b slots, the largest-remainder share of the
// n_splits * B slots by its key range len_b, so every slot of the batch has
// about sum(len) / (n_splits * B) keys; n_b is raised to
// ceil(len_b / keys_per_split) (no slot longer than the plan's) and to 1, and
// capped at n_slots, the workspace's slots per (sequence, KV head).  The
// sum of n_b is at most (n_splits + 1) * B.  Workgroup j takes the j-th
// (sequence, slot, KV head) triple; a workgroup past
// the last triple has nothing to do.  The triples run slot by slot (slot s of
// every sequence that has one, then slot s + 1), as with equal slots.  Every
// wave computes the same result (B <= 64: lane b holds sequence b).
struct Job {
  int b, g, slot, n_b, c;  // c: the sequence's context length (clamped)
};

__device__ __forceinline__ int64_t wave_sum_i64(int64_t x) {
#pragma unroll
  for (int off = 32; off > 0; off >>= 1) {
    const uint32_t lo = __shfl_xor(static_cast<uint32_t>(x), off, kWave);
    const uint32_t hi = __shfl_xor(static_cast<uint32_t>(static_cast<uint64_t>(x) >> 32), off, kWave);
    x += static_cast<int64_t>((static_cast<uint64_t>(hi) << 32) | lo);
  }
  return x;
}

__device__ bool balanced_job(const Plan &P, int j, int lane, Job *out) {
  const bool on = lane < P.B;
  int len = 0, c = 0;
  if (on) {
    c = min(max(P.ctx_lens[lane], 0), P.cap - P.N);
    const int lo = P.has_prefix ? 0 : c;
    const int hi = P.has_tree ? c + P.N : c;
    len = hi - lo;
  }
  const int64_t J = static_cast<int64_t>(P.n_splits) * P.B;
  const int64_t T = wave_sum_i64(len);
  int64_t fl = 0, rem = 0;
  if (T > 0) {
    // floor(num / T) through fp64: num < 2^44 and the quotient < 2^15, so
    // the truncated double quotient is off by at most one
    const int64_t num = static_cast<int64_t>(len) * J;
    fl = static_cast<int64_t>(static_cast<double>(num) / static_cast<double>(T));
    if (fl * T > num)
      --fl;
    else if ((fl + 1) * T <= num)
      ++fl;
    rem = num - fl * T;
  }
  const int64_t D = J - wave_sum_i64(fl);  // slots left for the largest remainders
  // rank of this lane's remainder among the non-empty sequences (ties by index)
  const bool elig = on && len > 0;
  int rank = 0;
  for (int m = 0; m < P.B; ++m) {
    const uint32_t rlo = __builtin_amdgcn_readlane(static_cast<uint32_t>(rem), m);
    const uint32_t rhi =
        __builtin_amdgcn_readlane(static_cast<uint32_t>(static_cast<uint64_t>(rem) >> 32), m);
    const int64_t rm = static_cast<int64_t>((static_cast<uint64_t>(rhi) << 32) | rlo);
    const bool em = __builtin_amdgcn_readlane(static_cast<int>(elig), m) != 0;
    rank += (em && (rm > rem || (rm == rem && m < lane))) ? 1 : 0;
  }
  int n = 0;
  if (on) {
    const int64_t lr = fl + ((elig && rank < D) ? 1 : 0);
    const int base = (len + P.keys_per_split - 1) / P.keys_per_split;
    n = static_cast<int>(min<int64_t>(max<int64_t>(max<int64_t>(lr, base), 1), P.n_slots));
  }
  // slot-major order: slot s of every sequence with n_b > s, KV heads inner
  int slot = 0, first = 0;
  uint64_t has;
  for (;;) {
    has = __ballot(n > slot);
    const int cnt = __popcll(has) * P.Hkv;
    if (cnt == 0) return false;
    if (j < first + cnt) break;
    first += cnt;
    ++slot;
  }
  const int r = j - first;
  const int idx = r / P.Hkv;  // the idx-th sequence (in order) with n_b > slot
  const uint32_t below = __builtin_amdgcn_mbcnt_hi(static_cast<uint32_t>(has >> 32),
                                                  __builtin_amdgcn_mbcnt_lo(static_cast<uint32_t>(has), 0u));
  const uint64_t pick = __ballot(((has >> lane) & 1) && static_cast<int>(below) == idx);
  const int b = __ffsll(static_cast<unsigned long long>(pick)) - 1;
  out->b = b;
  out->slot = slot;
  out->g = r - idx * P.Hkv;
  out->n_b = __builtin_amdgcn_readlane(n, b);
  out->c = __builtin_amdgcn_readlane(c, b);
  return true;
}

template <bool SPARSE, bool SPAGED>
__global__ __launch_bounds__(Cfg<waves_for(SPARSE)>::kNT, Cfg<waves_for(SPARSE)>::kWgPerCu)
void attn_partial_dma_small(Plan P) {
  using C = Cfg<waves_for(SPARSE)>;
  constexpr int kWaves = C::kWaves, kNT = C::kNT, kSmemBytes = C::kSmemBytes;
  constexpr int kIdxBytes = C::kIdxBytes, kEpiTpr = C::kEpiTpr, kEpiFeat = C::kEpiFeat;
  static_assert(SPARSE || !SPAGED, "paged gathers are sparse");
  __shared__ __attribute__((aligned(1024))) char smem[kSmemBytes + (SPAGED ? kTabBytes : 0)];

  const int tid = threadIdx.x;
  const int wave = __builtin_amdgcn_readfirstlane(tid / kWave);
  const int lane = tid % kWave;
  const int l32 = lane & 31, hf = lane >> 5;

  const int BH = P.B * P.Hkv;
  // A ragged dense batch takes balanced slots (the plan then has more slots
  // than splits); otherwise block j is slot j / BH of (sequence, KV head) j % BH.
  const bool balanced = !SPARSE && P.n_slots > P.n_splits;
  int b, g, slot, n_b, c;
  if (balanced) {
    Job jb;
    if (!balanced_job(P, blockIdx.x, lane, &jb)) return;
    b = jb.b;
    g = jb.g;
    slot = jb.slot;
    n_b = jb.n_b;
    c = jb.c;
  } else {
    slot = blockIdx.x / BH;
    b = (blockIdx.x % BH) / P.Hkv;
    g = (blockIdx.x % BH) % P.Hkv;
    n_b = P.n_splits;
    c = min(max(P.ctx_lens[b], 0), P.cap - P.N);
  }
  const int bg = b * P.Hkv + g;

  // ---- key range of this slot (prefix or index set, then draft rows) --------
  // Keys [0, cpos) are the prefix (dense: rows 0..c-1; sparse: rows
  // kv_idx[0..n_sel-1]), keys cpos + j are draft row c + j.
  const int cpos = SPARSE ? P.n_sel : c;
  const int lo = P.has_prefix ? 0 : cpos;
  const int hi = P.has_tree ? cpos + P.N : cpos;
  // Each sequence's own key range is cut into its n_b slots of equal length
  // (rounded up to whole 32-key blocks, 64 keys for a paged cache as the
  // plan's slots are), never longer than the plan's slot.  With equal
  // contexts the slots are the plan's.
  const int quantum = (!SPARSE && P.block_table != nullptr) ? 64 : kBK;
  const int len = hi - lo;
  const int kps = min(P.keys_per_split,
                      max(quantum, ((len + n_b - 1) / n_b + quantum - 1) / quantum * quantum));
  const int t_begin = lo + slot * kps;
  const int t_end = min(t_begin + kps, hi);
  const int n_blocks = t_end > t_begin ? (t_end - t_begin + kBK - 1) / kBK : 0;
  const int row_last = t_end - 1;
  const bool tree = t_end > cpos;
  const int mask_from = min(cpos, t_end);

  const int r = l32;  // this lane's grouped row
  const int64_t prow = (static_cast<int64_t>(slot) * BH + bg) * P.R + r;

  // Balanced slots: the workgroup of a sequence's last slot marks the
  // workspace slots n_b .. n_slots-1 of its (sequence, KV head) empty.  (Called
  // where no DMA is in flight: stores count in vmcnt too.)
  auto mark_unused = [&]() {
    if (balanced && slot == n_b - 1 && wave == 0 && hf == 0 && r < P.R)
      for (int s = n_b; s < P.n_slots; ++s) {
        const int64_t pr = (static_cast<int64_t>(s) * BH + bg) * P.R + r;
        P.lse_part[pr] = kNegInf;
        if (P.part_f16) P.o_scale[pr] = 1.f;
      }
  };

  if (n_blocks == 0) {
    if (wave == 0 && hf == 0 && r < P.R) {
      P.lse_part[prow] = kNegInf;
      if (P.part_f16) P.o_scale[prow] = 1.f;
    }
    mark_unused();
    return;
  }

  // this wave's blocks: i = wave, wave + kWaves, ...
  const int my_n = wave < n_blocks ? (n_blocks - wave + kWaves - 1) / kWaves : 0;

  const bool paged = !SPARSE && P.block_table != nullptr;
  const int64_t kv_row0 = (paged || SPAGED) ? 0 : static_cast<int64_t>(bg) * P.cap;
  const char *kbytes = static_cast<const char *>(P.k) + kv_row0 * kRowBytes;
  const char *vbytes = static_cast<const char *>(P.v) + kv_row0 * kRowBytes;
  // Paged cache (dense only): lane l holds the pool block of logical block
  // lb0 + l (a slot spans at most 33 blocks; 32-key blocks start at
  // multiples of 32 and pool blocks hold a power of two >= 64 rows, so a
  // key block lies in one pool block).  Entries outside the pool are
  // clamped into it.
  int lb0 = 0, ptab = 0;
  if (paged) {
    lb0 = t_begin >> P.block_shift;
    const int lb = lb0 + lane;
    const int nlb = ((t_end - 1) >> P.block_shift) - lb0 + 1;
    const int e = (lane < nlb && lb < P.max_blocks)
                      ? P.block_table[static_cast<int64_t>(b) * P.max_blocks + lb]
                      : 0;
    ptab = min(max(e, 0), P.n_pool_blocks - 1);
  }
  auto block_off = [&](const int row_first) -> int64_t {
    if (!paged) return static_cast<int64_t>(row_first) * kRowBytes;
    const int phys = __builtin_amdgcn_readlane(ptab, (row_first >> P.block_shift) - lb0);
    const int in_blk = row_first & ((1 << P.block_shift) - 1);
    return ((static_cast<int64_t>(phys) * P.Hkv + g) * (int64_t{1} << P.block_shift) + in_blk) *
           kRowBytes;
  };
  // Sparse over a paged cache: pool block of each logical block the rows
  // [0, c + N) fall in (c + N <= cap, and the plan admits at most
  // kTabEntries columns), clamped into the pool.
  const lds_i32 *tab = nullptr;
  if constexpr (SPAGED) {
    lds_i32 *t = (lds_i32 *)(smem + kSmemBytes);
    const int nb = (c + P.N + (1 << P.block_shift) - 1) >> P.block_shift;
    const int32_t *src = P.block_table + static_cast<int64_t>(b) * P.max_blocks;
    for (int j = tid; j < nb; j += kNT) t[j] = min(max(src[j], 0), P.n_pool_blocks - 1);
    __syncthreads();
    tab = t;
  }
  lds_char *const lds = (lds_char *)(smem);
  const uint32_t ring0 = static_cast<uint32_t>(reinterpret_cast<uintptr_t>(lds)) + wave * kWaveLds;

  // DMA lane offsets inside a block (K block kb: key (kb/4)*16 + lane%16,
  // chunk (kb%4)*4 + lane/16; V block vb: key (vb/4)*16 + lane/4, chunk
  // (vb%4)*4 + lane%4).
  auto k_key = [&](int kb) { return (kb >> 2) * 16 + (lane & 15); };
  auto k_chunk = [&](int kb) { return ((kb & 3) * 4 + (lane >> 4)) * 16; };
  auto v_key = [&](int vb) { return (vb >> 2) * 16 + (lane >> 2); };
  auto v_chunk = [&](int vb) { return ((vb & 3) * 4 + (lane & 3)) * 16; };

  // sparse: this wave's index ring, and the row-index fetch of its k-th block
  const int32_t *idx_row = SPARSE ? P.kv_idx + static_cast<int64_t>(bg) * P.n_sel : nullptr;
  const uint32_t iring0 = static_cast<uint32_t>(reinterpret_cast<uintptr_t>(lds)) +
                          (kSmemBytes - kIdxBytes) + wave * 2 * kIdxSlot;
  auto issue_idx = [&](const int k) {
    const int t0 = t_begin + (wave + kWaves * k) * kBK;
    const int t = min(t0 + (lane & 31), P.n_sel - 1);  // past the set: any valid index
    dma4(reinterpret_cast<const char *>(idx_row), static_cast<uint32_t>(t) * 4,
         iring0 + (k & 1) * kIdxSlot);
  };
  uint32_t vbits[2] = {~0u, ~0u};  // per-block validity (sparse), by k % 2

  // this wave's DMA of its k-th block into ring stage k % 2
  auto issue_block = [&](const int k) {
    if constexpr (SPARSE) {
      // rows of this lane's two K keys and two V keys, from the index ring
      const int t0 = t_begin + (wave + kWaves * k) * kBK;
      const int32_t *slot_idx =
          reinterpret_cast<const int32_t *>(smem + (kSmemBytes - kIdxBytes) +
                                            (wave * 2 + (k & 1)) * kIdxSlot);
      // Keys past the range's end and out-of-range indices are masked; they
      // load the row of the block's last key, which is in the key set (so its
      // values are finite: a masked key's probability is 0, and 0 * NaN would
      // still poison P.V).
      auto row_at = [&](int t) {  // cache row of key t < t_end, or -1
        if (t >= cpos) return c + (t - cpos);
        const int p = slot_idx[t - t0];
        return (p >= 0 && p < c) ? p : -1;
      };
      const int r_last = row_at(min(t0 + kBK, t_end) - 1);
      const int safe = r_last >= 0 ? r_last : 0;
      auto row_of = [&](int key) {
        const int t = t0 + key;
        const int rr = t < t_end ? row_at(t) : -1;
        return rr >= 0 ? rr : safe;
      };
      // validity of the block's 32 keys (lane j < 32 answers for key j)
      {
        const int t = t0 + (lane & 31);
        const int p = slot_idx[lane & 31];
        const bool ok = t < t_end && (t >= cpos || (p >= 0 && p < c));
        vbits[k & 1] = static_cast<uint32_t>(__ballot(ok));
      }
      const int rk0 = row_of(lane & 15), rk1 = row_of(16 + (lane & 15));
      const int rv0 = row_of(lane >> 2), rv1 = row_of(16 + (lane >> 2));
      const uint32_t st = ring0 + (k & 1) * kBlockBytes;
      if constexpr (SPAGED) {
        // cache row -> byte offset of its pool row (block, KV head g, row)
        const int sh = P.block_shift;
        auto pool_off = [&](const int row) -> int64_t {
          const int64_t blk = static_cast<int64_t>(tab[row >> sh]) * P.Hkv + g;
          return ((blk << sh) + (row & ((1 << sh) - 1))) * kRowBytes;
        };
        const char *kp0 = kbytes + pool_off(rk0), *kp1 = kbytes + pool_off(rk1);
        const char *vp0 = vbytes + pool_off(rv0), *vp1 = vbytes + pool_off(rv1);
#pragma unroll
        for (int x = 0; x < 8; ++x) {
          dma16p((x < 4 ? kp0 : kp1) + k_chunk(x), st + x * 1024);
          dma16p((x < 4 ? vp0 : vp1) + v_chunk(x), st + kHalfBytes + x * 1024);
        }
        return;
      }
#pragma unroll
      for (int x = 0; x < 8; ++x) {
        dma16(kbytes, static_cast<uint32_t>(x < 4 ? rk0 : rk1) * kRowBytes + k_chunk(x),
              st + x * 1024);
        dma16(vbytes, static_cast<uint32_t>(x < 4 ? rv0 : rv1) * kRowBytes + v_chunk(x),
              st + kHalfBytes + x * 1024);
      }
      return;
    }
    const int row_first = t_begin + (wave + kWaves * k) * kBK;
    const int lim = row_last - row_first;  // last valid key of the block
    const int64_t off = block_off(row_first);
    const char *kt = kbytes + off;
    const char *vt = vbytes + off;
    const uint32_t st = ring0 + (k & 1) * kBlockBytes;
    if (lim >= kBK - 1) {
#pragma unroll
      for (int x = 0; x < 8; ++x) {
        dma16(kt, k_key(x) * kRowBytes + k_chunk(x), st + x * 1024);
        dma16(vt, v_key(x) * kRowBytes + v_chunk(x), st + kHalfBytes + x * 1024);
      }
    } else {
#pragma unroll
      for (int x = 0; x < 8; ++x) {
        dma16(kt, min(k_key(x), lim) * kRowBytes + k_chunk(x), st + x * 1024);
        dma16(vt, min(v_key(x), lim) * kRowBytes + v_chunk(x), st + kHalfBytes + x * 1024);
      }
    }
  };

  // prologue: this wave's first two blocks, before the query loads.  Sparse:
  // indices of blocks 0 and 1, then blocks 0 and 1 with the indices of block
  // 2 between them, which is the order the loop keeps (see below).
  if constexpr (SPARSE) {
    if (my_n > 0) issue_idx(0);
    if (my_n > 1) issue_idx(1);
    wait_vm(0);
    if (my_n > 0) issue_block(0);
    if (my_n > 2) issue_idx(2);
    if (my_n > 1) issue_block(1);
  } else {
    if (my_n > 0) issue_block(0);
    if (my_n > 1) issue_block(1);
  }

  // ---- this lane's query (B operand of S^T = K.Q^T), tree mask word --------
  const uint4 *qv = static_cast<const uint4 *>(P.q);
  bf16x8 qf[8];
  uint64_t anc_q = 0;
  {
    const bool ok = r < P.R;
    const int i = ok ? r / P.G : 0;
    const int h = g * P.G + (ok ? r % P.G : 0);
    const int64_t qrow = (static_cast<int64_t>(b) * P.N + i) * P.Hq + h;
#pragma unroll
    for (int ks = 0; ks < 8; ++ks) {
      const uint4 u = ok ? qv[qrow * (kD / 8) + 2 * ks + hf] : make_uint4(0, 0, 0, 0);
      qf[ks] = __builtin_bit_cast(bf16x8, u);
    }
    if (tree) {
      if (P.anc) {
        anc_q = P.anc[static_cast<int64_t>(b) * P.N + i];
      } else {
        bool bad;
        const uint64_t a = tree_ancestors(P.parent + static_cast<int64_t>(b) * P.N, P.N, lane,
                                          &bad);
        anc_q = shfl_u64(a, i);
      }
    }
  }
  // Consume the query loads now; the compiler does not count the DMA, so its
  // wait is vmcnt(0) and the prologue blocks have landed too.
#pragma unroll
  for (int ks = 0; ks < 8; ++ks) asm volatile("" ::"v"(qf[ks]));
  asm volatile("" ::"v"(anc_q));

  const int k_base = (l32 >> 4) * 4096 + hf * 256 + (l32 & 15) * 16;
  const int g16 = lane >> 4, s16 = lane & 15;
  const int v_base = kHalfBytes + (4 * hf + (s16 >> 2)) * 64 +
                     (2 * (g16 & 1) + ((s16 & 3) >> 1)) * 16 + (s16 & 1) * 8;

  floatx16 o_acc[4];
#pragma unroll
  for (int db = 0; db < 4; ++db) o_acc[db] = floatx16{};
  float m_run = kNegInf, l_run = 0.f;
  const float cs = P.scale_log2;

  // Order of this wave's DMA: ..., data(k), [idx(k+2), data(k+1)], [idx(k+3),
  // data(k+2)], ...  so data(k) is complete once at most 16 * [k+1 < n] +
  // [k+2 < n] instructions are outstanding, and idx(k+2) once data(k+1)'s 16
  // are.
  for (int k = 0; k < my_n; ++k) {
    wait_vm((k + 1 < my_n ? 16 : 0) + (SPARSE && k + 2 < my_n ? 1 : 0));
    lds_char *const st = lds + wave * kWaveLds + (k & 1) * kBlockBytes;
    const int t0 = t_begin + (wave + kWaves * k) * kBK;

    // S^T = K . Q^T
    bf16x8 ka[8];
#pragma unroll
    for (int ks = 0; ks < 8; ++ks)
      ka[ks] = *(const lds_bf16x8 *)(st + k_base + (ks >> 1) * 1024 + (ks & 1) * 512);
    // V^T operands, needed after the softmax
    bf16x4 t4[4][2][2];
#pragma unroll
    for (int db = 0; db < 4; ++db)
#pragma unroll
      for (int half = 0; half < 2; ++half) {
        lds_char *vp = st + v_base + half * 4096 + db * 1024;
        t4[db][half][0] = __builtin_amdgcn_ds_read_tr16_b64_v4bf16((lds_bf16x4 *)(vp));
        t4[db][half][1] = __builtin_amdgcn_ds_read_tr16_b64_v4bf16((lds_bf16x4 *)(vp + 512));
      }
    floatx16 sv = floatx16{};
#pragma unroll
    for (int ks = 0; ks < 8; ++ks)
      sv = __builtin_amdgcn_mfma_f32_32x32x16_bf16(ka[ks], qf[ks], sv, 0, 0, 0);

    // mask: keys past the slot's end, draft rows by ancestor bits, invalid
    // indices (lane value e is key t0 + 4*hf + 8*(e/4) + e%4)
    const uint32_t vb = SPARSE ? vbits[k & 1] : ~0u;
    if (t0 + kBK > mask_from || vb != ~0u) {
      const int base = t0 + 4 * hf;
      const int room = t_end - base;
      const int pre = cpos - base;
      uint32_t keep = pre <= 0 ? 0u : pre >= 32 ? ~0u : ((1u << pre) - 1u);
      if (tree) {
        const int sh = -pre;
        keep |= sh >= 64 || sh <= -32 ? 0u
                : sh >= 0         ? static_cast<uint32_t>(anc_q >> sh)
                                  : static_cast<uint32_t>(anc_q << (-sh));
      }
      keep &= room <= 0 ? 0u : room >= 32 ? ~0u : ((1u << room) - 1u);
      keep &= vb >> (4 * hf);
#pragma unroll
      for (int e = 0; e < 16; ++e) {
        const int bit = 8 * (e >> 2) + (e & 3);
        sv[e] = ((keep >> bit) & 1u) ? sv[e] : kNegInf;
      }
    }

    // softmax against the running reference (fast path), exact fp32 sum
    float p[16];
    float sum = 0.f;
#pragma unroll
    for (int e = 0; e < 16; ++e) {
      p[e] = fast_exp2(fmaf(sv[e], cs, -m_run));
      sum += p[e];
    }
    bf16x8 pb[2];
#pragma unroll
    for (int half = 0; half < 2; ++half) {
      floatx8 x;
#pragma unroll
      for (int e = 0; e < 8; ++e) x[e] = p[8 * half + e];
      pb[half] = __builtin_convertvector(x, bf16x8);
    }
    // keep the conversion ahead of the branch (see attn_dma.hip)
    asm volatile("" : "+v"(pb[0]), "+v"(pb[1]));
    if (__builtin_expect(__any(!(sum <= kSumLimit) || m_run == kNegInf), 0)) {
      float mx = kNegInf;
#pragma unroll
      for (int e = 0; e < 16; ++e) mx = fmaxf(mx, sv[e]);
      mx = fmaxf(mx, __shfl_xor(mx, 32, kWave)) * cs;
      const float m_new = fmaxf(m_run, mx);
      const float m_use = m_new == kNegInf ? 0.f : m_new;
      const float alpha = fast_exp2(m_run - m_use);
      sum = 0.f;
#pragma unroll
      for (int e = 0; e < 16; ++e) {
        p[e] = fast_exp2(fmaf(sv[e], cs, -m_use));
        sum += p[e];
      }
#pragma unroll
      for (int half = 0; half < 2; ++half) {
        floatx8 x;
#pragma unroll
        for (int e = 0; e < 8; ++e) x[e] = p[8 * half + e];
        pb[half] = __builtin_convertvector(x, bf16x8);
      }
      if (__any(m_run != kNegInf && alpha != 1.f)) {
#pragma unroll
        for (int db = 0; db < 4; ++db) o_acc[db] *= alpha;
      }
      l_run *= alpha;
      m_run = m_new;
    }
    l_run += sum;

    // O^T += V^T . P^T
#pragma unroll
    for (int db = 0; db < 4; ++db)
#pragma unroll
      for (int half = 0; half < 2; ++half) {
        const bf16x8 a = __builtin_shufflevector(t4[db][half][0], t4[db][half][1], 0, 1, 2, 3, 4,
                                                 5, 6, 7);
        o_acc[db] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, pb[half], o_acc[db], 0, 0, 0);
      }

    // refill this stage with block k+2 once its operands have been read
    // (the index fetch of block k+3 reuses the slot of block k+1, whose rows
    // were read before block k+1 was issued)
    if (k + 2 < my_n) {
      asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
      if constexpr (SPARSE) {
        wait_vm(16);  // idx(k+2) has landed
        if (k + 3 < my_n) issue_idx(k + 3);
      }
      issue_block(k + 2);
    }
  }

  // ---- merge the waves' results through LDS ---------------------------------
  // Each wave's row statistics (log2-domain reference and sum) and its
  // unnormalised accumulator rows; then every thread combines 16 values of
  // one row: weights 2^(m_w - M) / L with L = sum_w l_w 2^(m_w - M).
  const float l_tot = l_run + __shfl_xor(l_run, 32, kWave);
  __syncthreads();  // every wave is done with its ring
  mark_unused();
  float *stat_m = reinterpret_cast<float *>(smem + kWaves * kRows * kEpiRow);
  float *stat_l = stat_m + kWaves * kRows;
  if (hf == 0) {
    stat_m[wave * kRows + l32] = l_tot > 0.f ? m_run : kNegInf;
    stat_l[wave * kRows + l32] = l_tot;
  }
  char *ep = smem + wave * kRows * kEpiRow;
#pragma unroll
  for (int db = 0; db < 4; ++db)
#pragma unroll
    for (int jj = 0; jj < 4; ++jj) {
      float4 v4;
      v4.x = o_acc[db][4 * jj + 0];
      v4.y = o_acc[db][4 * jj + 1];
      v4.z = o_acc[db][4 * jj + 2];
      v4.w = o_acc[db][4 * jj + 3];
      *reinterpret_cast<float4 *>(ep + l32 * kEpiRow + (32 * db + 8 * jj + 4 * hf) * 4) = v4;
    }
  __syncthreads();

  // thread -> (row, kEpiFeat features): kEpiTpr threads per row, rows 0..31
  const int row = tid / kEpiTpr, f0 = (tid % kEpiTpr) * kEpiFeat;
  float mw[kWaves], lw[kWaves];
  float M = kNegInf;
#pragma unroll
  for (int w = 0; w < kWaves; ++w) {
    mw[w] = stat_m[w * kRows + row];
    lw[w] = stat_l[w * kRows + row];
    M = fmaxf(M, mw[w]);
  }
  float L = 0.f, sc[kWaves];
#pragma unroll
  for (int w = 0; w < kWaves; ++w) {
    sc[w] = mw[w] == kNegInf ? 0.f : fast_exp2(mw[w] - M);
    L += lw[w] * sc[w];
  }
  const float inv = L > 0.f ? 1.f / L : 0.f;
  float o16[kEpiFeat];
#pragma unroll
  for (int e = 0; e < kEpiFeat; ++e) o16[e] = 0.f;
#pragma unroll
  for (int w = 0; w < kWaves; ++w) {
    const float wt = sc[w] * inv;
    const float *src = reinterpret_cast<const float *>(smem + (w * kRows + row) * kEpiRow) + f0;
#pragma unroll
    for (int e = 0; e < kEpiFeat; ++e) o16[e] = fmaf(wt, src[e], o16[e]);
  }
  if (!P.part_f16) {
    // fp32 partial rows (HSV_FLAG_F32_PARTIALS)
    if (row < P.R) {
      const int64_t orow = (static_cast<int64_t>(slot) * BH + bg) * P.R + row;
      float *dst = P.o_part + orow * kD + f0;
#pragma unroll
      for (int e = 0; e < kEpiFeat; e += 4)
        *reinterpret_cast<float4 *>(dst + e) = make_float4(o16[e], o16[e + 1], o16[e + 2],
                                                           o16[e + 3]);
      if (tid % kEpiTpr == 0) P.lse_part[orow] = L > 0.f ? (M + fast_log2(L)) * kLn2 : kNegInf;
    }
    return;
  }
  // scaled fp16: the row's largest |value| in [0.5, 1), scale to o_scale
  float amax = 0.f;
#pragma unroll
  for (int e = 0; e < kEpiFeat; ++e) amax = fmaxf(amax, fabsf(o16[e]));
#pragma unroll
  for (int off = 1; off < kEpiTpr; off <<= 1) amax = fmaxf(amax, __shfl_xor(amax, off, kWave));
  int ex = 0;
  if (amax > 0.f && amax < __builtin_huge_valf()) (void)frexpf(amax, &ex);
  const float mul = ldexpf(1.f, -ex);
  if (row < P.R) {
    const int64_t orow = (static_cast<int64_t>(slot) * BH + bg) * P.R + row;
    _Float16 *dst = reinterpret_cast<_Float16 *>(P.o_part) + orow * kD + f0;
#pragma unroll
    for (int e0 = 0; e0 < kEpiFeat; e0 += 8) {
      halfx8 h;
#pragma unroll
      for (int e = 0; e < 8; ++e) h[e] = static_cast<_Float16>(o16[e0 + e] * mul);
      *reinterpret_cast<halfx8 *>(dst + e0) = h;
    }
    if (tid % kEpiTpr == 0) {
      P.lse_part[orow] = L > 0.f ? (M + fast_log2(L)) * kLn2 : kNegInf;
      P.o_scale[orow] = ldexpf(1.f, ex);
    }
  }
}

}  // namespace

bool dma_small_supports(const Plan &p) {
  // sparse DMA offsets are 32-bit byte offsets from the (b, kv head) base
  return p.in_dtype == kBF16 && p.D == kD && p.R <= kRows &&
         (p.n_sel == 0 || static_cast<int64_t>(p.cap) * kRowBytes < (int64_t{1} << 32));
}

// the planner's slot unit: a slot is split further while longer than 64 of these
int dma_small_tile_keys() { return 4 * kBK; }
int dma_small_wgs_per_cu(bool sparse) {
  return sparse ? Cfg<waves_for(true)>::kWgPerCu : Cfg<waves_for(false)>::kWgPerCu;
}

int dma_small_table_entries() { return kTabEntries; }

hipError_t launch_attn_partials_dma_small(const Plan &p, hipStream_t s) {
  // balanced slots (n_slots > n_splits): at most (n_splits + 1) * B triples per KV head
  const int64_t grid_slots = p.n_slots > p.n_splits ? p.n_splits + 1 : p.n_slots;
  const int64_t blocks = grid_slots * p.B * p.Hkv;
  if (p.n_sel > 0 && p.block_table)
    hipLaunchKernelGGL((attn_partial_dma_small<true, true>), dim3(static_cast<unsigned>(blocks)),
                       dim3(Cfg<waves_for(true)>::kNT), 0, s, p);
  else if (p.n_sel > 0)
    hipLaunchKernelGGL((attn_partial_dma_small<true, false>), dim3(static_cast<unsigned>(blocks)),
                       dim3(Cfg<waves_for(true)>::kNT), 0, s, p);
  else
    hipLaunchKernelGGL((attn_partial_dma_small<false, false>), dim3(static_cast<unsigned>(blocks)),
                       dim3(Cfg<waves_for(false)>::kNT), 0, s, p);
  return hipGetLastError();
}

}  // namespace hsv
