// Partial verification attention for 256-row query groups with a direct
// HBM -> LDS pipeline (gfx950).
//
// Same arithmetic as attn_mfma.hip (S^T = K.Q^T and O^T += V^T.P^T on
// v_mfma_f32_32x32x16_bf16, one lane per query, online softmax in the log2
// domain); what differs is how K and V reach the matrix cores:
//
//  * global_load_lds_dwordx4 moves each 16-byte chunk straight into LDS (no
//    staging registers), so a workgroup keeps kAhead tiles of 64 keys in
//    flight while it computes on another -- the memory-level parallelism the
//    HBM stream needs.
//  * Each DMA instruction fills 1 KB: 16 keys x 4 consecutive 16-byte chunks.
//    A tile is 16 such blocks for K and 16 for V, block b = (key/16)*4 +
//    chunk/4.  Inside a K block the order is (chunk%4)*256 + (key%16)*16, so
//    each 16-lane quarter of a K operand read covers 256 contiguous bytes;
//    inside a V block it is (key%16)*64 + (chunk%4)*16, so each half-wave of
//    a transpose read covers 256 contiguous bytes.  Every LDS read below is
//    one lane base register plus an immediate.
//  * The DMA addresses are a scalar base (the tile's first cache row) plus a
//    per-lane 32-bit byte offset that is the same for every full tile, so
//    issuing a tile costs no vector address arithmetic.
//  * V stays row-major in LDS; the V^T operand of P.V comes from
//    ds_read_b64_tr_b16, which hands each lane of a 16-lane group one b16
//    element from each of four other lanes' 8-byte rows: lane s of a group
//    points at V[k0 + s/4][d0 + 4(s%4) .. +3] and lane i receives
//    V[k0 + j][d0 + i], j = 0..3 -- four consecutive keys of one feature.
//  * The DMA is issued from inline assembly, so the compiler neither counts it
//    nor guards LDS reads against it; waits are explicit instead: one asm
//    statement does s_waitcnt vmcnt(n) for this thread's own DMA and then
//    s_barrier, with a memory clobber so no LDS access moves across it.  No
//    full memory fence, so later tiles stay in flight.  The query rows take
//    the same DMA path (into two stages that tiles 2 and 3 reuse later), so
//    the first tiles are in flight with them from the start.  M0 (the LDS
//    base of the DMA) is set inside the same asm statement; the kernel uses
//    M0 for nothing else.
//  * The V^T operands of a key block are read before its softmax, so their
//    LDS latency overlaps the exponentials.
//
// Rows of keys outside the slot are fetched from the slot's last valid row
// (so every address is inside the cache and every staged value is a real,
// finite cache entry) and masked out of the softmax.
#include "common.hpp"
#include "launch.h"

namespace hsv {
namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef float floatx16 __attribute__((ext_vector_type(16)));
typedef float floatx8 __attribute__((ext_vector_type(8)));
typedef float floatx4 __attribute__((ext_vector_type(4)));
typedef float floatx2 __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef _Float16 halfx4 __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) char lds_char;
typedef __attribute__((address_space(3))) bf16x4 lds_bf16x4;
typedef __attribute__((address_space(3))) bf16x8 lds_bf16x8;

constexpr int kNW = 8;              // waves: 8 x 32 query rows
constexpr int kNT = kNW * 64;
constexpr int kTK = 64;             // keys per tile
constexpr int kD = 128;
constexpr int kRowBytes = kD * 2;   // one bf16 cache row
constexpr int kTileBytes = kTK * kRowBytes;    // 16 KB (K or V)
constexpr int kStageBytes = 2 * kTileBytes;    // K then V
constexpr int kStages = 4;
constexpr int kAhead = 2;           // tiles in flight beyond the one computed on
// The DMA of tile j+1+kAhead is issued while block 2j+1 (tile j) is still
// being computed, so its stage must differ from those of tiles j and j+1.
static_assert(kAhead + 2 <= kStages, "stage of the refilled tile is still being read");
constexpr int kBlocks = kTileBytes / 1024;     // 1 KB DMA blocks per K (or V) tile
constexpr int kBlocksPerWave = kBlocks / kNW;  // per wave, for K and again for V
constexpr int kDmaPerTile = 2 * kBlocksPerWave;  // DMA instructions per thread per tile
// Epilogue staging: every wave's 32 x 128 fp16 partial, rows padded by 16 B.
constexpr int kEpiRowStride = kD * 2 + 16;
// Query staging: the workgroup's 256 query rows (64 KB) in stages 2 and 3,
// which the tiles first reuse after the first barrier.  Inside a row, 16-byte
// chunk c sits at position c ^ (row % 16), so a 16-lane read of one chunk
// from 16 rows touches 16 distinct bank groups.
constexpr int kQOff = 2 * kStageBytes;
static_assert(kQOff + kNW * 32 * kRowBytes <= kStages * kStageBytes, "query staging");
static_assert(kAhead == 2, "the prologue issues tiles 0 and 1 with the query");
constexpr int kSmemBytes = kStages * kStageBytes > kNW * 32 * kEpiRowStride
                               ? kStages * kStageBytes
                               : kNW * 32 * kEpiRowStride;

// Largest per-lane sum of 16 probabilities the fast softmax path accepts
// (each probability then stays <= 2^16, far from fp32/bf16 overflow).
constexpr float kSumLimit = 65536.f;

// 16 bytes per lane from global memory straight into LDS at lds_base + 16*lane
// (lds_base is wave-uniform and goes through M0).  Address = sbase + voff.
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
#pragma clang diagnostic pop

// Wait until this thread's DMA of the current tile is done (the next tile's
// may still be in flight), then meet the other waves: their DMA of the
// current tile is then in LDS too, and they are done reading the stage the
// next DMA will overwrite.
// `later` = tiles issued after the current one (0 .. kAhead - 1 outstanding
// beyond it).
__device__ __forceinline__ void wait_tile_and_sync(int later) {
  static_assert(kDmaPerTile == 4, "the immediates below assume 4 DMA ops per tile");
  static_assert(kAhead <= 3, "immediates below");
  if (later >= 2)
    asm volatile("s_waitcnt vmcnt(8)\n\ts_barrier" ::: "memory");
  else if (later == 1)
    asm volatile("s_waitcnt vmcnt(4)\n\ts_barrier" ::: "memory");
  else
    asm volatile("s_waitcnt vmcnt(0)\n\ts_barrier" ::: "memory");
}

__global__ __launch_bounds__(kNT, 1) void attn_partial_dma(Plan P) {
  __shared__ __attribute__((aligned(1024))) char smem[kSmemBytes];
  // the ancestor mask of each of this workgroup's rows, as 32-bit words
  // (word w holds draft nodes 32w .. 32w+31; zero past the tree's words)
  __shared__ uint32_t wide_mask[kNW * 32 * 8];

  const int tid = threadIdx.x;
  const int wave = __builtin_amdgcn_readfirstlane(tid / kWave);
  const int lane = tid % kWave;
  const int l32 = lane & 31, hf = lane >> 5;

  // Workgroup -> (row chunk rc, unit = slot * B * Hkv + bg).  Consecutive
  // workgroups go to the eight XCDs in turn, each with an L2 of its own.  The
  // row chunks of one unit read the same K/V tiles at about the same time, so
  // when a unit has several they go to one XCD (workgroups bid, bid + 8, ...)
  // and all but the first find the tiles in its L2.  A unit count that is not
  // a multiple of eight keeps the plain order.
  const int bid = blockIdx.x;
  int rc, unit;
  if (P.row_chunks > 1 && (gridDim.x / P.row_chunks) % 8 == 0) {
    const int xcd = bid % 8, k = bid / 8;
    rc = k % P.row_chunks;
    unit = (k / P.row_chunks) * 8 + xcd;
  } else {
    rc = bid % P.row_chunks;
    unit = bid / P.row_chunks;
  }
  const int BH = P.B * P.Hkv;
  const int bg = unit % BH;
  const int slot = unit / BH;
  const int b = bg / P.Hkv, g = bg % P.Hkv;

  // ---- key range of this slot: cache rows [t_begin, t_end) -----------------
  // The prefix rows [0, c) and the draft rows [c, c + N) form one range
  // [lo, hi); rows at or past c are visible to a query only through its
  // ancestor bits.
  const int c = min(max(P.ctx_lens[b], 0), P.cap - P.N);
  const int lo = P.has_prefix ? 0 : c;
  const int hi = P.has_tree ? c + P.N : c;
  const int t_begin = lo + slot * P.keys_per_split;
  const int t_end = min(t_begin + P.keys_per_split, hi);
  const int n_tiles = t_end > t_begin ? (t_end - t_begin + kTK - 1) / kTK : 0;
  const int row_last = t_end - 1;      // last valid row: clamp target
  const bool tree = t_end > c;         // the range reaches the draft rows
  const int mask_from = min(c, t_end); // blocks reaching past this row are masked

  const int row_base = rc * (kNW * 32) + wave * 32;
  const int r = row_base + l32;
  const int part = slot;  // one key group: one partial per slot
  const int64_t prow = (static_cast<int64_t>(part) * BH + bg) * P.R + r;

  if (n_tiles == 0) {
    if (r < P.R && hf == 0) {
      P.lse_part[prow] = kNegInf;
      if (P.part_f16) P.o_scale[prow] = 1.f;
    }
    return;
  }

  // byte bases of this (batch, kv head)'s cache rows
  const bool paged = P.block_table != nullptr;
  const int64_t kv_row0 = paged ? 0 : static_cast<int64_t>(bg) * P.cap;
  const char *kbytes = static_cast<const char *>(P.k) + kv_row0 * kRowBytes;
  const char *vbytes = static_cast<const char *>(P.v) + kv_row0 * kRowBytes;
  // Paged cache: lane l holds the pool block of logical block lb0 + l (a
  // slot spans at most 33 blocks; tiles start at multiples of 64 keys and
  // blocks hold a power of two >= 64 rows, so a tile lies in one block).
  // Entries outside the pool are clamped into it.
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
  // first-row byte offset of the tile starting at cache row row_first
  auto tile_off = [&](const int row_first) -> int64_t {
    if (!paged) return static_cast<int64_t>(row_first) * kRowBytes;
    const int phys = __builtin_amdgcn_readlane(ptab, (row_first >> P.block_shift) - lb0);
    const int in_blk = row_first & ((1 << P.block_shift) - 1);
    return ((static_cast<int64_t>(phys) * P.Hkv + g) * (int64_t{1} << P.block_shift) + in_blk) *
           kRowBytes;
  };
  // C-style cast: the generic -> LDS address-space conversion
  lds_char *const lds = (lds_char *)(smem);
  const uint32_t lds0 = static_cast<uint32_t>(reinterpret_cast<uintptr_t>(lds));

  // ---- DMA of one tile --------------------------------------------------------
  // K block blk: lane i carries key (blk/4)*16 + i%16, chunk (blk%4)*4 + i/16;
  // V block blk: key (blk/4)*16 + i/4, chunk (blk%4)*4 + i%4.
  // The lane offsets are recomputed for every tile (a few VALU operations)
  // rather than held in registers through the main loop.
  // This thread's DMA of tile j into stage j % kStages.
  auto issue_tile = [&](const int j) {
    const int row_first = t_begin + j * kTK;
    const int lim = row_last - row_first;  // last valid key of the tile
    const int64_t off = tile_off(row_first);
    const char *kt = kbytes + off;
    const char *vt = vbytes + off;
    const uint32_t st = lds0 + (j % kStages) * kStageBytes;
    int ln = lane;
    asm volatile("" : "+v"(ln));  // not hoisted out of the loop
    const bool full = lim >= kTK - 1;
#pragma unroll
    for (int bw = 0; bw < kBlocksPerWave; ++bw) {
      const int blk = wave * kBlocksPerWave + bw;
      const uint32_t blk_off = blk * 1024;
      const int krel = (blk >> 2) * 16 + (ln & 15);
      const int vrel = (blk >> 2) * 16 + (ln >> 2);
      const uint32_t kch = ((blk & 3) * 4 + (ln >> 4)) * 16;
      const uint32_t vch = ((blk & 3) * 4 + (ln & 3)) * 16;
      dma16(kt, (full ? krel : min(krel, lim)) * kRowBytes + kch, st + blk_off);
      dma16(vt, (full ? vrel : min(vrel, lim)) * kRowBytes + vch, st + kTileBytes + blk_off);
    }
  };

  // prologue: this wave's 32 query rows, then tiles 0 and 1, all by DMA, so
  // the first tiles need not wait for the query to land.  Each 1 KB DMA
  // instruction carries four rows; lane l takes chunk (l % 16) ^ (row % 16)
  // of row 4j + l / 16, which lands at position l % 16 of that row.  Rows
  // past R fetch row 0 of the group (a real entry) and are zeroed on reading.
  // The paged block table is read first (issue_tile needs it), so no
  // compiler wait for it covers the query DMA.
  asm volatile("" ::"v"(ptab));
  {
    const char *qb = static_cast<const char *>(P.q) +
                     static_cast<int64_t>(b) * P.N * P.Hq * kRowBytes;
    const uint32_t qlds = lds0 + kQOff + (wave * 32) * kRowBytes;
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      const int rw = 4 * j + (lane >> 4);  // row inside the wave's 32
      const int rr = row_base + rw;
      const int rv = rr < P.R ? rr : 0;
      const int qi = rv / P.G, qh = g * P.G + rv % P.G;
      const uint32_t off = static_cast<uint32_t>((qi * P.Hq + qh) * kRowBytes) +
                           static_cast<uint32_t>((((lane & 15) ^ (rw & 15))) * 16);
      dma16(qb, off, qlds + j * 1024);
    }
  }
  issue_tile(0);
  if (n_tiles > 1) issue_tile(1);
  // the query DMA was issued first: it has landed once at most the tiles'
  // four (or eight) instructions are outstanding
  if (n_tiles > 1)
    asm volatile("s_waitcnt vmcnt(8)" ::: "memory");
  else
    asm volatile("s_waitcnt vmcnt(4)" ::: "memory");

  // ---- this lane's query (B operand of S^T = K.Q^T), tree mask word --------
  bf16x8 qf[8];
  {
    const bool ok = r < P.R;
    const int i = ok ? r / P.G : 0;
    lds_char *const qrow_lds = lds + kQOff + (wave * 32 + l32) * kRowBytes;
#pragma unroll
    for (int ks = 0; ks < 8; ++ks) {
      const bf16x8 x = *(const lds_bf16x8 *)(qrow_lds + (((2 * ks + hf) ^ (l32 & 15)) * 16));
      qf[ks] = ok ? x : bf16x8{};
    }
    if (tree && P.anc_words > 1) {
      // rows of this workgroup: their masks into LDS (zero past R)
      const int rl = tid / 2;  // 512 threads: two per row, alternate words
      const int rr = rc * (kNW * 32) + rl;
      const int ii = rr < P.R ? rr / P.G : 0;
      const uint64_t *src = P.anc + (static_cast<int64_t>(b) * P.N + ii) * P.anc_words;
      for (int w = tid & 1; w < 4; w += 2) {
        const uint64_t x = (rr < P.R && w < P.anc_words) ? src[w] : 0;
        wide_mask[rl * 8 + 2 * w] = static_cast<uint32_t>(x);
        wide_mask[rl * 8 + 2 * w + 1] = static_cast<uint32_t>(x >> 32);
      }
    } else if (tree) {
      // one 64-bit word per row: this wave's rows into the same LDS layout
      // (words 2..7 zero), written and read by this wave only
      uint64_t anc_q;
      if (P.anc) {
        anc_q = P.anc[static_cast<int64_t>(b) * P.N + i];
      } else {
        bool bad;
        const uint64_t a = tree_ancestors(P.parent + static_cast<int64_t>(b) * P.N, P.N, lane,
                                          &bad);
        anc_q = shfl_u64(a, i);
      }
      uint32_t *mw = wide_mask + (wave * 32 + l32) * 8 + 4 * hf;
      mw[0] = hf == 0 ? static_cast<uint32_t>(anc_q) : 0u;
      mw[1] = hf == 0 ? static_cast<uint32_t>(anc_q >> 32) : 0u;
      mw[2] = 0u;
      mw[3] = 0u;
    }
  }

  // Consume the query (and tree) reads now: every wave is done with the
  // query staging before the first barrier, after which tile 2 reuses it.
  // (Tree masks are read with ordinary loads, which the compiler waits for
  // with vmcnt(0), tiles 0 and 1 included; only the workgroups whose keys
  // reach the draft rows read them.)
#pragma unroll
  for (int ks = 0; ks < 8; ++ks) asm volatile("" ::"v"(qf[ks]));
  // the LDS mask words of wide trees are read by every wave (this barrier's
  // wait for all memory operations costs nothing: the mask loads above
  // already wait for everything in flight)
  if (tree && P.anc_words > 1) __syncthreads();

  // lane bases of the LDS reads (byte offsets inside a stage)
  const int k_base = (l32 >> 4) * 4096 + hf * 256 + (l32 & 15) * 16;
  const int g16 = lane >> 4, s16 = lane & 15;
  const int v_base = kTileBytes + (4 * hf + (s16 >> 2)) * 64 +
                     (2 * (g16 & 1) + ((s16 & 3) >> 1)) * 16 + (s16 & 1) * 8;

  floatx16 o_acc[4];
#pragma unroll
  for (int db = 0; db < 4; ++db) o_acc[db] = floatx16{};
  float m_run = kNegInf, l_run = 0.f;
  const float cs = P.scale_log2;

  // K operands of one 32-key block (block kb of the tile in stage st), and
  // S^T = K . Q^T from them.
  auto read_k = [&](lds_char *const st, const int kb, bf16x8 (&ka)[8]) {
#pragma unroll
    for (int ks = 0; ks < 8; ++ks)
      ka[ks] = *(const lds_bf16x8 *)(st + k_base + kb * 8192 + (ks >> 1) * 1024 + (ks & 1) * 512);
  };
  auto qk_mfma = [&](const bf16x8 (&ka)[8], floatx16 &sv) {
    sv = floatx16{};
#pragma unroll
    for (int ks = 0; ks < 8; ++ks)
      sv = __builtin_amdgcn_mfma_f32_32x32x16_bf16(ka[ks], qf[ks], sv, 0, 0, 0);
  };

  // V^T operands of key block kb (two transpose reads per operand).
  auto read_v = [&](lds_char *const st, const int kb, bf16x8 (&va)[4][2]) {
    bf16x4 t[4][2][2];
#pragma unroll
    for (int db = 0; db < 4; ++db)
#pragma unroll
      for (int half = 0; half < 2; ++half) {
        lds_char *vp = st + v_base + (kb * 2 + half) * 4096 + db * 1024;
        t[db][half][0] = __builtin_amdgcn_ds_read_tr16_b64_v4bf16((lds_bf16x4 *)(vp));
        t[db][half][1] = __builtin_amdgcn_ds_read_tr16_b64_v4bf16((lds_bf16x4 *)(vp + 512));
      }
#pragma unroll
    for (int db = 0; db < 4; ++db)
#pragma unroll
      for (int half = 0; half < 2; ++half)
        va[db][half] = __builtin_shufflevector(t[db][half][0], t[db][half][1], 0, 1, 2, 3, 4, 5,
                                               6, 7);
  };

  // The half `half` (keys 16*half .. +15 of the block) of the V^T operands.
  auto read_v_half = [&](lds_char *const st, const int kb, const int half, bf16x8 (&va)[4][2]) {
#pragma unroll
    for (int db = 0; db < 4; ++db) {
      lds_char *vp = st + v_base + (kb * 2 + half) * 4096 + db * 1024;
      const bf16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4bf16((lds_bf16x4 *)(vp));
      const bf16x4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4bf16((lds_bf16x4 *)(vp + 512));
      va[db][half] = __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7);
    }
  };

  auto to_bf16 = [&](const float (&p)[16], bf16x8 (&pb)[2]) {
#pragma unroll
    for (int half = 0; half < 2; ++half) {
      floatx8 x;
#pragma unroll
      for (int e = 0; e < 8; ++e) x[e] = p[8 * half + e];
      pb[half] = __builtin_convertvector(x, bf16x8);
    }
  };

  // Mask of one 32-key block (cache rows t0 .. t0+31).  Lane value e holds
  // key t0 + 4*hf + 8*(e/4) + e%4, i.e. bit 8*(e/4) + e%4 of a 32-bit word
  // whose bit i is key t0 + 4*hf + i.
  auto apply_mask = [&](floatx16 &sv, const int t0) {
    const int base = t0 + 4 * hf;
    const int room = t_end - base;  // keys inside the slot
    const int pre = c - base;       // prefix keys (always visible)
    uint32_t keep = pre <= 0 ? 0u : pre >= 32 ? ~0u : ((1u << pre) - 1u);
    if (tree) {
      // bits [sh, sh + 32) of this row's N-bit mask, from the LDS words
      const int sh = -pre;
      const int a = sh >= 0 ? sh / 32 : -((31 - sh) / 32);  // floor(sh / 32)
      const int o = sh - 32 * a;
      const uint32_t *mw = wide_mask + (wave * 32 + l32) * 8;
      const uint32_t lo = (a >= 0 && a < 8) ? mw[a] : 0u;
      const uint32_t hi = (a + 1 >= 0 && a + 1 < 8) ? mw[a + 1] : 0u;
      keep |= static_cast<uint32_t>(((static_cast<uint64_t>(hi) << 32) | lo) >> o);
    }
    keep &= room <= 0 ? 0u : room >= 32 ? ~0u : ((1u << room) - 1u);
#pragma unroll
    for (int e = 0; e < 16; ++e) {
      const int bit = 8 * (e >> 2) + (e & 3);
      sv[e] = ((keep >> bit) & 1u) ? sv[e] : kNegInf;
    }
  };

  // Probabilities of one block against the running reference m_run (log2
  // domain), as bf16 B operands, and their exact fp32 sum.  No branches: this
  // is the work that overlaps the next block's QK^T MFMAs.
  auto fast_p = [&](const floatx16 &sv, bf16x8 (&pb)[2]) {
    float p[16];
    float sum = 0.f;
#pragma unroll
    for (int e = 0; e < 16; ++e) {
      p[e] = fast_exp2(fmaf(sv[e], cs, -m_run));
      sum += p[e];
    }
    to_bf16(p, pb);
    return sum;
  };

  // Slow path of the softmax: the block maximum becomes the new reference,
  // the accumulators are rescaled and the block's probabilities recomputed.
  // Taken when a lane's 16 probabilities sum above kSumLimit (a key well
  // above the reference) or nothing has been visible yet.  The normalised
  // result does not depend on the reference.
  auto slow_p = [&](const floatx16 &sv, bf16x8 (&pb)[2], float &sum) {
    float mx = kNegInf;
#pragma unroll
    for (int e = 0; e < 16; ++e) mx = fmaxf(mx, sv[e]);
    mx = fmaxf(mx, __shfl_xor(mx, 32, kWave)) * cs;
    const float m_new = fmaxf(m_run, mx);
    const float m_use = m_new == kNegInf ? 0.f : m_new;
    const float alpha = fast_exp2(m_run - m_use);  // 0 when m_run = -inf
    float p[16];
    sum = 0.f;
#pragma unroll
    for (int e = 0; e < 16; ++e) {
      p[e] = fast_exp2(fmaf(sv[e], cs, -m_use));
      sum += p[e];
    }
    to_bf16(p, pb);
    if (__any(m_run != kNegInf && alpha != 1.f)) {
#pragma unroll
      for (int db = 0; db < 4; ++db) o_acc[db] *= alpha;
    }
    l_run *= alpha;
    m_run = m_new;
  };

  // O^T += V^T . P^T for one key block.
  auto pv = [&](const bf16x8 (&va)[4][2], const bf16x8 (&pb)[2]) {
#pragma unroll
    for (int db = 0; db < 4; ++db)
#pragma unroll
      for (int half = 0; half < 2; ++half)
        o_acc[db] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(va[db][half], pb[half], o_acc[db], 0,
                                                            0, 0);
  };

  // Software pipeline over 32-key blocks t = 0 .. 2*n_tiles - 1 (block t is
  // half t % 2 of tile t / 2).  Step t computes block t's probabilities
  // while the matrix cores run the QK^T MFMAs of block t+1 and the P.V MFMAs
  // of block t-1, alternating, so a wave keeps both the VALU and the matrix
  // core busy and no MFMA waits on the one before it.  Every LDS read of a
  // step is consumed inside that step.  Tile j sits in stage j % kStages;
  // the barrier of step 2j+1 (before the first read of tile j+1) also tells
  // every wave that the others are done with step 2j, the last reader of
  // tile j-1, whose stage the DMA of tile j+1+kAhead then reuses.  The last
  // step's "next block" reads a stage that holds an older tile: its scores
  // are never used.
  //
  // The probabilities of block t are taken against the running reference
  // m_run; when the slow path moves the reference, the accumulators already
  // hold P.V of blocks up to t-1 and are rescaled with l_run, and block t's
  // probabilities (carried to step t+1 in pb_prev) use the new reference.
  // 32-key blocks holding keys of the slot; a slot of an odd number of
  // blocks ends in a half tile whose second block is not computed
  const int n_blocks = (t_end - t_begin + 31) / 32;
  const int s_mask = kStages * kStageBytes - 1;
  // stage byte offset of block tb's tile (stage sizes are a power of two)
  auto stage_of = [&](const int tb) { return lds + (((tb >> 1) * kStageBytes) & s_mask); };
  bf16x8 pb_prev[2];

  auto step = [&](const int t, floatx16 &s_cur, floatx16 &s_nxt, auto with_pv) {
    constexpr bool kPV = decltype(with_pv)::value;
    const int t0 = t_begin + t * 32;
    // the next block's K operands, then the previous block's V^T operands
    bf16x8 ka[8];
    read_k(stage_of(t + 1), (t + 1) & 1, ka);
    // V^T operands: the first halves now, the second halves (used by the
    // last four P.V MFMAs) from the third MFMA pair on, to bound the live
    // registers
    bf16x8 va[4][2];
    lds_char *const vst = stage_of(t - 1);
    const int vkb = (t - 1) & 1;
    if constexpr (kPV) read_v_half(vst, vkb, 0, va);
    if (t0 + 32 > mask_from) apply_mask(s_cur, t0);
    uint32_t pw[8];  // probabilities 2w, 2w+1 as a bf16 pair
    float sum = 0.f;
    s_nxt = floatx16{};
#pragma unroll
    for (int ks = 0; ks < 8; ++ks) {
      s_nxt = __builtin_amdgcn_mfma_f32_32x32x16_bf16(ka[ks], qf[ks], s_nxt, 0, 0, 0);
      if constexpr (kPV) {
        if (ks == 2) read_v_half(vst, vkb, 1, va);
      }
      if constexpr (kPV)
        o_acc[ks & 3] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(va[ks & 3][ks >> 2],
                                                                pb_prev[ks >> 2], o_acc[ks & 3],
                                                                0, 0, 0);
      floatx2 x;
      x[0] = fast_exp2(fmaf(s_cur[2 * ks], cs, -m_run));
      x[1] = fast_exp2(fmaf(s_cur[2 * ks + 1], cs, -m_run));
      sum += x[0];
      sum += x[1];
      pw[ks] = __builtin_bit_cast(uint32_t, __builtin_convertvector(x, bf16x2));
    }
    // Issue order: a few exponentials while the K operands arrive, then each
    // QK^T MFMA and each P.V MFMA followed by three VALU operations, and the
    // second half of the V^T reads after the third pair.
    __builtin_amdgcn_sched_group_barrier(0x002, 4, 0);
#pragma unroll
    for (int ks = 0; ks < 8; ++ks) {
      __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
      __builtin_amdgcn_sched_group_barrier(0x002, 3, 0);
      if constexpr (kPV) {
        __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
        __builtin_amdgcn_sched_group_barrier(0x002, 3, 0);
        if (ks == 2) __builtin_amdgcn_sched_group_barrier(0x100, 8, 0);
      }
    }
    bf16x8 pb[2];
    pb[0] = __builtin_bit_cast(bf16x8, make_uint4(pw[0], pw[1], pw[2], pw[3]));
    pb[1] = __builtin_bit_cast(bf16x8, make_uint4(pw[4], pw[5], pw[6], pw[7]));
    // Keep the conversion ahead of the branch: otherwise the compiler sinks
    // it into the fast path, the fp32 probabilities stay live across the
    // join with the slow path, and the merge copies registers (spills, whose
    // scratch loads would also wait on the DMA in flight).
    asm volatile("" : "+v"(pb[0]), "+v"(pb[1]));
    if (__builtin_expect(__any(!(sum <= kSumLimit) || m_run == kNegInf), 0))
      slow_p(s_cur, pb, sum);
    l_run += sum;
    pb_prev[0] = pb[0];
    pb_prev[1] = pb[1];
  };
  using no_pv = std::integral_constant<bool, false>;
  using has_pv = std::integral_constant<bool, true>;

  wait_tile_and_sync(min(n_tiles - 1, kAhead - 1));
  if (kAhead < n_tiles) issue_tile(kAhead);
  floatx16 s_a, s_b;  // scores of the even and the odd blocks
  {
    bf16x8 ka[8];
    read_k(lds, 0, ka);
    qk_mfma(ka, s_a);
  }
  step(0, s_a, s_b, no_pv{});
  for (int j = 0; j + 1 < n_tiles; ++j) {
    // step 2j+1 reads the K operands of tile j+1
    wait_tile_and_sync(min(n_tiles - 2 - j, kAhead - 1));
    if (j + 1 + kAhead < n_tiles) issue_tile(j + 1 + kAhead);
    step(2 * j + 1, s_b, s_a, has_pv{});
    step(2 * j + 2, s_a, s_b, has_pv{});
  }
  // an odd block count ends inside the loop (its last step is the first
  // block of the last tile)
  if (!(n_blocks & 1)) step(n_blocks - 1, s_b, s_a, has_pv{});
  {
    // P.V of the last block
    bf16x8 va[4][2];
    read_v(stage_of(n_blocks - 1), (n_blocks - 1) & 1, va);
    pv(va, pb_prev);
  }

  // ---- epilogue --------------------------------------------------------------
  // The normalised partial row of a query is written as fp16 scaled by a
  // power of two: its largest |value| lands in [0.5, 1), the scale 2^e goes
  // to o_scale (exact), and every value keeps 11 significant bits -- half
  // the bytes of fp32 for the write here and the merge's read.  The rows are
  // staged through LDS (lane l holds a query column; rows padded by 16 bytes
  // so the column-wise writes spread over banks) so the global stores are
  // whole 256-byte rows.
  const float l_tot = l_run + __shfl_xor(l_run, 32, kWave);
  const float inv = l_tot > 0.f ? 1.f / l_tot : 0.f;
  float amax = 0.f;
#pragma unroll
  for (int db = 0; db < 4; ++db)
#pragma unroll
    for (int e = 0; e < 16; ++e) amax = fmaxf(amax, fabsf(o_acc[db][e]));
  amax = fmaxf(amax, __shfl_xor(amax, 32, kWave)) * inv;
  int ex = 0;
  if (amax > 0.f && amax < __builtin_huge_valf()) (void)frexpf(amax, &ex);
  const float mul = ldexpf(inv, -ex);
  if (hf == 0 && r < P.R) {
    P.lse_part[prow] = l_tot > 0.f ? (m_run + fast_log2(l_tot)) * kLn2 : kNegInf;
    if (P.part_f16) P.o_scale[prow] = ldexpf(1.f, ex);
  }
  if (!P.part_f16) {
    // fp32 partial rows (HSV_FLAG_F32_PARTIALS) straight from the
    // accumulators: each lane stores four consecutive features at a time
    if (r < P.R) {
      float *dst = P.o_part + prow * kD + 4 * hf;
#pragma unroll
      for (int db = 0; db < 4; ++db)
#pragma unroll
        for (int jj = 0; jj < 4; ++jj) {
          floatx4 v4;
#pragma unroll
          for (int q = 0; q < 4; ++q) v4[q] = o_acc[db][4 * jj + q] * inv;
          *reinterpret_cast<floatx4 *>(dst + 32 * db + 8 * jj) = v4;
        }
    }
    return;
  }
  __syncthreads();  // every wave is done with the K/V stages
  char *ep = smem + wave * 32 * kEpiRowStride;
#pragma unroll
  for (int db = 0; db < 4; ++db)
#pragma unroll
    for (int jj = 0; jj < 4; ++jj) {
      floatx4 v4;
#pragma unroll
      for (int q = 0; q < 4; ++q) v4[q] = o_acc[db][4 * jj + q] * mul;
      *reinterpret_cast<halfx4 *>(ep + l32 * kEpiRowStride + (32 * db + 8 * jj + 4 * hf) * 2) =
          __builtin_convertvector(v4, halfx4);
    }
  __builtin_amdgcn_wave_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQ_REL, "wavefront");
  // row row_base of this wave, fp16
  char *dst0 = reinterpret_cast<char *>(P.o_part) + (prow - l32) * kD * 2;
#pragma unroll
  for (int it = 0; it < 8; ++it) {
    const int row = 4 * it + (lane >> 4);  // four rows per instruction
    const uint4 v = *reinterpret_cast<const uint4 *>(ep + row * kEpiRowStride + (lane & 15) * 16);
    if (row_base + row < P.R)
      *reinterpret_cast<uint4 *>(dst0 + row * kD * 2 + (lane & 15) * 16) = v;
  }
}

}  // namespace

// The kernel writes its partials in the scaled fp16 format (part_f16), or in
// fp32 when the caller asks for it.
bool dma_supports(const Plan &p) {
  return p.in_dtype == kBF16 && p.D == kD && p.n_sel == 0 && p.R > 128;
}

int dma_rows_per_wg() { return kNW * 32; }
int dma_tile_keys() { return kTK; }

hipError_t launch_attn_partials_dma(const Plan &p, hipStream_t s) {
  const int64_t blocks = static_cast<int64_t>(p.n_slots) * p.B * p.Hkv * p.row_chunks;
  hipLaunchKernelGGL(attn_partial_dma, dim3(static_cast<unsigned>(blocks)), dim3(kNT), 0, s, p);
  return hipGetLastError();
}

}  // namespace hsv
