// Partial verification attention for 256-row query groups with a direct
// HBM -> LDS pipeline (gfx950).
//
// Same arithmetic as attn_mfma.hip (S^T = K.Q^T and O^T += V^T.P^T on
// v_mfma_f32_32x32x16_bf16, one lane per query, online softmax in the log2
// domain); what differs is how K and V reach the matrix cores:
//
//  * global_load_lds_dwordx4 moves each 16-byte chunk straight into LDS (no
//    staging registers), so a workgroup keeps two tiles of 64 keys in
//    flight while it computes on another -- the memory-level parallelism the
//    HBM stream needs (prefetch distance two; see the main loop for why).
//  * Each DMA instruction fills 1 KB: 16 keys x 4 consecutive 16-byte chunks.
//    A tile is 16 such blocks for K and 16 for V, block b = (key/16)*4 +
//    chunk/4.  Inside a K block the order is (chunk%4)*256 + (key%16)*16, so
//    each 16-lane quarter of a K operand read covers 256 contiguous bytes;
//    inside a V block it is (key%16)*64 + (chunk%4)*16, so each half-wave of
//    a transpose read covers 256 contiguous bytes.  Every LDS read below is
//    one lane base register plus an immediate.
//  * V stays row-major in LDS; the V^T operand of P.V comes from
//    ds_read_b64_tr_b16, which hands each lane of a 16-lane group one b16
//    element from each of four other lanes' 8-byte rows: lane s of a group
//    points at V[k0 + s/4][d0 + 4(s%4) .. +3] and lane i receives
//    V[k0 + j][d0 + i], j = 0..3 -- four consecutive keys of one feature.
//  * The DMA is issued from inline assembly, so the compiler neither counts it
//    nor guards LDS reads against it; waits are explicit instead: one asm
//    statement does s_waitcnt vmcnt(n) for this thread's own DMA and then
//    s_barrier, with a memory clobber so no LDS access moves across it.  No
//    full memory fence, so later tiles stay in flight.  The query loads are
//    consumed before the first DMA is issued, so the compiler's own vmcnt
//    waits never cover an unknown DMA count.  M0 (the LDS base of the DMA) is
//    set inside the same asm statement; the kernel uses M0 for nothing else.
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
typedef __attribute__((address_space(3))) char lds_char;
typedef __attribute__((address_space(3))) bf16x4 lds_bf16x4;

constexpr int kNW = 8;              // waves: 8 x 32 query rows
constexpr int kNT = kNW * 64;
constexpr int kTK = 64;             // keys per tile
constexpr int kD = 128;
constexpr int kCH = kD / 8;         // 16-byte chunks per row
constexpr int kTileBytes = kTK * kD * 2;       // 16 KB (K or V)
constexpr int kStageBytes = 2 * kTileBytes;    // K then V
constexpr int kStages = 4;
constexpr int kBlocks = kTileBytes / 1024;     // 1 KB DMA blocks per K (or V) tile
constexpr int kBlocksPerWave = kBlocks / kNW;  // per wave, for K and again for V
constexpr int kDmaPerTile = 2 * kBlocksPerWave;  // DMA instructions per thread per tile
// Epilogue staging: every wave's 32 x 128 fp32 partial, rows padded by 16 B.
constexpr int kEpiRowStride = kD * 4 + 16;
constexpr int kSmemBytes = kStages * kStageBytes > kNW * 32 * kEpiRowStride
                               ? kStages * kStageBytes
                               : kNW * 32 * kEpiRowStride;

// Largest per-lane sum of 16 probabilities the fast softmax path accepts
// (each probability then stays <= 2^16, far from fp32/bf16 overflow).
constexpr float kSumLimit = 65536.f;

// 16 bytes per lane from global memory straight into LDS at `lds` + 16*lane
// (the LDS base is wave-uniform and goes through M0).
__device__ __forceinline__ void dma16(const void *gptr, lds_char *lds) {
  const uint32_t base = __builtin_amdgcn_readfirstlane(
      static_cast<uint32_t>(reinterpret_cast<uintptr_t>(lds)));
  asm volatile(
      "s_mov_b32 m0, %1\n\t"
      "s_nop 0\n\t"
      "global_load_lds_dwordx4 %0, off"
      :
      : "v"(gptr), "s"(base)
      : "memory", "m0");
}

// This thread's DMA of one tile: kBlocksPerWave K blocks and as many V blocks.
__device__ __forceinline__ void issue_tile(const uint4 *kc, const uint4 *vc, int row_first,
                                           int row_last, int lane, int wave, lds_char *stage) {
#pragma unroll
  for (int bw = 0; bw < kBlocksPerWave; ++bw) {
    const int blk = wave * kBlocksPerWave + bw;
    // K block: (chunk%4)*256 + (key%16)*16 -- lane i: key i%16, chunk i/16
    const int kkey = (blk >> 2) * 16 + (lane & 15);
    const int kchunk = (blk & 3) * 4 + (lane >> 4);
    const int krow = min(row_first + kkey, row_last);
    dma16(kc + static_cast<int64_t>(krow) * kCH + kchunk, stage + blk * 1024);
    // V block: (key%16)*64 + (chunk%4)*16 -- lane i: key i/4, chunk i%4
    const int vkey = (blk >> 2) * 16 + (lane >> 2);
    const int vchunk = (blk & 3) * 4 + (lane & 3);
    const int vrow = min(row_first + vkey, row_last);
    dma16(vc + static_cast<int64_t>(vrow) * kCH + vchunk, stage + kTileBytes + blk * 1024);
  }
}

// Wait until this thread's DMA of the current tile is done (the next tile's
// may still be in flight), then meet the other waves: their DMA of the
// current tile is then in LDS too, and they are done reading the stage the
// next DMA will overwrite.
__device__ __forceinline__ void wait_tile_and_sync(bool next_in_flight) {
  static_assert(kDmaPerTile == 4, "the immediate below assumes 4 DMA ops per tile");
  if (next_in_flight)
    asm volatile("s_waitcnt vmcnt(4)\n\ts_barrier" ::: "memory");
  else
    asm volatile("s_waitcnt vmcnt(0)\n\ts_barrier" ::: "memory");
}

__global__ __launch_bounds__(kNT, 1) void attn_partial_dma(Plan P) {
  __shared__ __attribute__((aligned(1024))) char smem[kSmemBytes];
  static_assert(kStages == 4, "tile j+2 is fetched while tiles j-1, j, j+1 stay resident");

  const int tid = threadIdx.x;
  const int wave = tid / kWave, lane = tid % kWave;
  const int l32 = lane & 31, hf = lane >> 5;

  int bid = blockIdx.x;
  const int rc = bid % P.row_chunks;
  bid /= P.row_chunks;
  const int BH = P.B * P.Hkv;
  const int bg = bid % BH;
  const int slot = bid / BH;
  const int b = bg / P.Hkv, g = bg % P.Hkv;
  const bool tree = slot == P.tree_slot;

  // ---- key range of this slot: cache rows [row_lo + t] for t in [t_begin, t_end)
  const int c = min(max(P.ctx_lens[b], 0), P.cap - P.N);
  int t_begin, t_end, row_off;
  if (tree) {
    t_begin = 0;
    t_end = P.N;
    row_off = c;
  } else {
    t_begin = slot * P.keys_per_split;
    t_end = min(t_begin + P.keys_per_split, c);
    row_off = 0;
  }
  const int n_tiles = t_end > t_begin ? (t_end - t_begin + kTK - 1) / kTK : 0;
  const int row_last = row_off + t_end - 1;  // last valid row: clamp target

  const int row_base = rc * (kNW * 32) + wave * 32;
  const int r = row_base + l32;
  const int part = slot;  // one key group: one partial per slot
  const int64_t prow = (static_cast<int64_t>(part) * BH + bg) * P.R + r;

  if (n_tiles == 0) {
    if (r < P.R && hf == 0) P.lse_part[prow] = kNegInf;
    return;
  }

  const int64_t kv_row0 = static_cast<int64_t>(bg) * P.cap;
  const uint4 *kc = static_cast<const uint4 *>(P.k) + kv_row0 * kCH;
  const uint4 *vc = static_cast<const uint4 *>(P.v) + kv_row0 * kCH;
  // C-style cast: the generic -> LDS address-space conversion
  lds_char *const lds = (lds_char *)(smem);

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
      const uint4 u = ok ? qv[qrow * kCH + 2 * ks + hf] : make_uint4(0, 0, 0, 0);
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

  // Consume the query (and tree) loads now: the compiler's wait for them then
  // happens before the first DMA is in flight.
#pragma unroll
  for (int ks = 0; ks < 8; ++ks) asm volatile("" ::"v"(qf[ks]));
  asm volatile("" ::"v"(anc_q));

  // prologue: tiles 0 and 1 in flight (prefetch distance two)
  issue_tile(kc, vc, row_off + t_begin, row_last, lane, wave, lds);
  if (n_tiles > 1) issue_tile(kc, vc, row_off + t_begin + kTK, row_last, lane, wave, lds + kStageBytes);

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

  // S^T = K . Q^T for the two 32-key blocks of the tile in stage `st`; all K
  // operands are read first so the LDS latency overlaps the matrix work.
  auto qk = [&](lds_char *const st, floatx16 (&sv)[2]) {
    bf16x8 ka[2][8];
#pragma unroll
    for (int kb = 0; kb < 2; ++kb)
#pragma unroll
      for (int ks = 0; ks < 8; ++ks)
        ka[kb][ks] = *reinterpret_cast<const __attribute__((address_space(3))) bf16x8 *>(
            st + k_base + kb * 8192 + (ks >> 1) * 1024 + (ks & 1) * 512);
#pragma unroll
    for (int kb = 0; kb < 2; ++kb) {
      sv[kb] = floatx16{};
#pragma unroll
      for (int ks = 0; ks < 8; ++ks)
        sv[kb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(ka[kb][ks], qf[ks], sv[kb], 0, 0, 0);
    }
  };

  // Mask and softmax of one 32-key block (keys kb0 .. kb0+31 of a tile with
  // nv valid keys); returns the block's P^T as two bf16 B operands.
  auto softmax = [&](floatx16 &sv, const int kb0, const int nv, bf16x8 (&pb)[2]) {
    if (tree || kb0 + 32 > nv) {
      const int room = nv - kb0 - 4 * hf;
      uint32_t keep = room <= 0 ? 0u : room >= 32 ? ~0u : ((1u << room) - 1u);
      if (tree) {
        const int sh = kb0 + 4 * hf;
        keep &= sh < 64 ? static_cast<uint32_t>(anc_q >> sh) : 0u;
      }
#pragma unroll
      for (int e = 0; e < 16; ++e) {
        const int bit = 8 * (e >> 2) + (e & 3);
        sv[e] = ((keep >> bit) & 1u) ? sv[e] : kNegInf;
      }
    }
    // Probabilities against the running reference m_run (log2 domain).
    // Fast path: no block maximum; if the lane's 16 probabilities sum above
    // kSumLimit (a key well above the reference) or nothing is visible yet,
    // the wave takes the slow path: block maximum, new reference, rescale.
    // The normalised result does not depend on the reference.
    float pv[16];
    float sum = 0.f;
#pragma unroll
    for (int e = 0; e < 16; ++e) {
      pv[e] = fast_exp2(fmaf(sv[e], cs, -m_run));
      sum += pv[e];
    }
    if (__builtin_expect(__any(!(sum <= kSumLimit) || m_run == kNegInf), 0)) {
      float mx = kNegInf;
#pragma unroll
      for (int e = 0; e < 16; ++e) mx = fmaxf(mx, sv[e]);
      mx = fmaxf(mx, __shfl_xor(mx, 32, kWave)) * cs;
      const float m_new = fmaxf(m_run, mx);
      const float m_use = m_new == kNegInf ? 0.f : m_new;
      const float alpha = fast_exp2(m_run - m_use);  // 0 when m_run = -inf
      sum = 0.f;
#pragma unroll
      for (int e = 0; e < 16; ++e) {
        pv[e] = fast_exp2(fmaf(sv[e], cs, -m_use));
        sum += pv[e];
      }
      if (__any(m_run != kNegInf && alpha != 1.f)) {
#pragma unroll
        for (int db = 0; db < 4; ++db) o_acc[db] *= alpha;
      }
      l_run *= alpha;
      m_run = m_new;
    }
    l_run += sum;
#pragma unroll
    for (int half = 0; half < 2; ++half) {
      floatx8 x;
#pragma unroll
      for (int e = 0; e < 8; ++e) x[e] = pv[8 * half + e];
      pb[half] = __builtin_convertvector(x, bf16x8);
    }
  };

  // O^T += V^T . P^T for key block kb of the tile in stage `st`; V^T
  // operands come from transpose reads (two per operand), all read first.
  auto pv = [&](lds_char *const st, const int kb, const bf16x8 (&pb)[2]) {
    bf16x4 va[4][2][2];
#pragma unroll
    for (int db = 0; db < 4; ++db)
#pragma unroll
      for (int half = 0; half < 2; ++half) {
        lds_char *vp = st + v_base + (kb * 2 + half) * 4096 + db * 1024;
        va[db][half][0] = __builtin_amdgcn_ds_read_tr16_b64_v4bf16((lds_bf16x4 *)(vp));
        va[db][half][1] = __builtin_amdgcn_ds_read_tr16_b64_v4bf16((lds_bf16x4 *)(vp + 512));
      }
#pragma unroll
    for (int db = 0; db < 4; ++db)
#pragma unroll
      for (int half = 0; half < 2; ++half) {
        const bf16x8 a = __builtin_shufflevector(va[db][half][0], va[db][half][1], 0, 1, 2, 3, 4,
                                                 5, 6, 7);
        o_acc[db] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, pb[half], o_acc[db], 0, 0, 0);
      }
  };

  // The two waves sharing a SIMD (w and w + 4) run half a tile apart: the
  // lagging half finishes the previous tile's second key block (softmax on
  // the VALU, then P.V) while the leading half starts the new tile with its
  // QK^T MFMAs, so one wave's VALU work overlaps the other's matrix work
  // instead of both alternating in lock-step after every barrier.  The
  // prefetch distance is two tiles, so the previous tile's stage is still
  // intact while the lagging waves read it.
  const bool lag = wave >= kNW / 2;
  floatx16 s_keep = floatx16{};
  int nv_keep = 0;
  for (int j = 0; j < n_tiles; ++j) {
    wait_tile_and_sync(j + 1 < n_tiles);
    if (j + 2 < n_tiles)
      issue_tile(kc, vc, row_off + t_begin + (j + 2) * kTK, row_last, lane, wave,
                 lds + ((j + 2) % kStages) * kStageBytes);
    lds_char *const st = lds + (j % kStages) * kStageBytes;
    const int nv = min(kTK, t_end - (t_begin + j * kTK));
    if (lag && j > 0) {
      bf16x8 pb[2];
      softmax(s_keep, 32, nv_keep, pb);
      pv(lds + ((j - 1) % kStages) * kStageBytes, 1, pb);
    }
    floatx16 sv[2];
    qk(st, sv);
    {
      bf16x8 pb[2];
      softmax(sv[0], 0, nv, pb);
      pv(st, 0, pb);
    }
    if (lag) {
      s_keep = sv[1];
      nv_keep = nv;
    } else {
      bf16x8 pb[2];
      softmax(sv[1], 32, nv, pb);
      pv(st, 1, pb);
    }
  }
  if (lag) {
    bf16x8 pb[2];
    softmax(s_keep, 32, nv_keep, pb);
    pv(lds + ((n_tiles - 1) % kStages) * kStageBytes, 1, pb);
  }

  // ---- epilogue --------------------------------------------------------------
  // Normalise, then write the wave's 32 x 128 partial through LDS so that the
  // global stores are whole 512-byte rows (lane l holds a query column; rows
  // are padded by 16 bytes so the column-wise LDS writes spread over banks).
  const float l_tot = l_run + __shfl_xor(l_run, 32, kWave);
  const float inv = l_tot > 0.f ? 1.f / l_tot : 0.f;
  if (hf == 0 && r < P.R)
    P.lse_part[prow] = l_tot > 0.f ? (m_run + fast_log2(l_tot)) * kLn2 : kNegInf;
  constexpr int kRowStride = kEpiRowStride;
  __syncthreads();  // every wave is done with the K/V stages
  char *ep = smem + wave * 32 * kRowStride;
#pragma unroll
  for (int db = 0; db < 4; ++db)
#pragma unroll
    for (int jj = 0; jj < 4; ++jj) {
      float4 v4;
      v4.x = o_acc[db][4 * jj + 0] * inv;
      v4.y = o_acc[db][4 * jj + 1] * inv;
      v4.z = o_acc[db][4 * jj + 2] * inv;
      v4.w = o_acc[db][4 * jj + 3] * inv;
      *reinterpret_cast<float4 *>(ep + l32 * kRowStride + (32 * db + 8 * jj + 4 * hf) * 4) = v4;
    }
  __builtin_amdgcn_wave_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQ_REL, "wavefront");
  float *dst0 = P.o_part + (prow - l32) * kD;  // row row_base of this wave
#pragma unroll
  for (int it = 0; it < 16; ++it) {
    const int row = 2 * it + (lane >> 5);  // two rows per instruction
    const float4 v4 = *reinterpret_cast<const float4 *>(ep + row * kRowStride + (lane & 31) * 16);
    if (row_base + row < P.R)
      *reinterpret_cast<float4 *>(dst0 + row * kD + (lane & 31) * 4) = v4;
  }
}

}  // namespace

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
