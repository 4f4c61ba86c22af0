// Partial verification attention on the bf16 matrix cores (gfx950 MFMA).
//
// One workgroup (4 waves) owns one slot of one (sequence b, KV head g): a
// contiguous range of prefix keys (LongSpec section 2.C, cache part, no
// mask), the same over gathered index-set rows (Dustin page, verification
// over the selected subset), or the draft block under the ancestor mask
// (the speculative part).  It streams that key range from HBM in tiles of
// TK keys, staged through LDS and shared by the waves, so every K/V byte is
// read once per KV head for all G*N grouped query rows.
//
// Matrix layout ("transposed" so that one lane owns one query throughout):
//   S^T[key][q] = K[key][:] . Q[q][:]    v_mfma_f32_32x32x16_bf16, A = K tile
//                                        rows from LDS, B = Q^T (registers)
//   O^T[d][q]  += V^T[d][key] . P^T[key][q]   A = V^T from LDS, B = P^T,
//                                        taken straight from the S^T
//                                        accumulators after the softmax.
// The 32x32 accumulator gives lane l the query column l%32 and the rows
// 8j + 4(l/32) + r (j, r in 0..3), so the online-softmax statistics of a
// query live in one lane pair (l, l^32) and need one cross-half exchange.
// V is written to LDS transposed, with keys permuted (bits 2 and 3 of the key
// index swapped inside each 16-key group) so that the eight keys a lane needs
// for one P.V step are contiguous and come in as one 16-byte LDS read.
// K rows and V^T rows are padded by 16 bytes against bank conflicts.  Waves are arranged as RG row groups x KG key groups; each wave
// writes its own partial (KG partials per slot), merged later with the rest.
#include "common.hpp"
#include "launch.h"

namespace hsv {
namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float floatx16 __attribute__((ext_vector_type(16)));
typedef float floatx8 __attribute__((ext_vector_type(8)));

template <int D_, int NW_, int KG_, int QB_, int KBW_>
struct Cfg {
  static constexpr int D = D_;
  static constexpr int NW = NW_;             // waves per workgroup
  static constexpr int NT = NW_ * 64;        // threads per workgroup
  static constexpr int KG = KG_;             // waves along keys
  static constexpr int RG = NW_ / KG_;       // waves along rows
  static constexpr int QB = QB_;             // 32-query blocks per wave
  static constexpr int KBW = KBW_;           // 32-key blocks per wave per tile
  static constexpr int TK = 32 * KBW * KG;   // keys per tile
  static constexpr int ROWS = RG * QB * 32;  // grouped rows per workgroup
  static constexpr int CH = D / 8;           // 16-byte chunks per K/V row
  static constexpr int DK = D / 16;          // MFMA k-steps over the features
  static constexpr int DB = D / 32;          // 32-feature blocks of O
  // LDS rows are padded by 16 bytes: 8 lanes reading the same 16-byte column
  // of 8 consecutive rows then hit 8 different 4-bank groups, and every
  // unrolled read is one base register plus an immediate offset.
  static constexpr int KSTRIDE = D * 2 + 16;                // bytes per K row
  static constexpr int VSTRIDE = TK * 2 + 16;               // bytes per V^T row
  static constexpr int K_BYTES = TK * KSTRIDE;
  static constexpr int V_BYTES = D * VSTRIDE;
  static constexpr int BUF_BYTES = K_BYTES + V_BYTES;
  static constexpr int NKL = (TK * CH + NT - 1) / NT;       // K loads per thread
  static constexpr int NVG = (TK / 4 * CH + NT - 1) / NT;   // 4-key V groups per thread
};

// Largest gap (log2 units) between a block maximum and the running softmax
// reference before the reference moves: probabilities stay <= 2^8.
constexpr float kSlack = 8.f;

__device__ __forceinline__ int swap_bits23(int k) {
  return (k & ~12) | ((k & 4) << 1) | ((k & 8) >> 1);
}

__device__ __forceinline__ uint32_t pack_lo(uint32_t a, uint32_t b) {
  return __builtin_amdgcn_perm(b, a, 0x05040100u);  // (b.lo << 16) | a.lo
}
__device__ __forceinline__ uint32_t pack_hi(uint32_t a, uint32_t b) {
  return __builtin_amdgcn_perm(b, a, 0x07060302u);  // (b.hi << 16) | a.hi
}

template <class C>
struct Tile {
  uint4 k[C::NKL];
  uint4 v[C::NVG][4];
};

// The keys of one slot: key t (t in [0, t_end)) is cache row idx[t] (sparse
// prefix) or row off + t (dense prefix: off = 0; draft block: off = c).
struct KeySource {
  int off;
  int t_end;
  int c;                 // sparse rows must lie in [0, c)
  const int32_t *idx;    // NULL unless a sparse prefix slot
};

// Cache row of key t, or -1 when the key does not exist (past the slot's end
// or an out-of-range index).  Never reads outside idx[0, t_end).
__device__ __forceinline__ int index_row(const KeySource &src, int t) {
  if (t >= src.t_end) return -1;
  const int p = src.idx[t];
  return (p >= 0 && p < src.c) ? p : -1;
}

// Cache row of key t0 + k.  A sparse slot's rows come from the tile's row
// table in LDS (filled from the index list two tiles ahead, so the data loads
// never wait on an index load); a dense slot's rows are contiguous.
template <bool SPARSE>
__device__ __forceinline__ int key_row(const KeySource &src, const int32_t *rows, int t0, int k) {
  if (SPARSE && src.idx) return rows[k];
  const int t = t0 + k;
  return t < src.t_end ? src.off + t : -1;
}

// Branch-free 16-byte load: invalid rows read row 0 of this (b, kv head) and
// are replaced by zeros, so masked keys never carry NaN or stale data.
__device__ __forceinline__ uint4 load_row_chunk(const uint4 *base, int row, int ch, int ch_per_row) {
  const uint4 x = base[static_cast<int64_t>(row < 0 ? 0 : row) * ch_per_row + ch];
  return row < 0 ? make_uint4(0, 0, 0, 0) : x;
}

template <class C, bool SPARSE>
__device__ __forceinline__ void load_tile(Tile<C> &tl, const uint4 *kc, const uint4 *vc,
                                          const KeySource &src, const int32_t *rows, int t0,
                                          int tid) {
  if (!(SPARSE && src.idx) && t0 + C::TK <= src.t_end) {
    // a whole tile of contiguous rows: no per-key checks
    const int row0 = src.off + t0;
#pragma unroll
    for (int i = 0; i < C::NKL; ++i) {
      const int item = tid + C::NT * i;
      if (C::TK * C::CH % C::NT != 0 && item >= C::TK * C::CH) break;
      tl.k[i] = kc[static_cast<int64_t>(row0 + item / C::CH) * C::CH + item % C::CH];
    }
#pragma unroll
    for (int i = 0; i < C::NVG; ++i) {
      const int item = tid + C::NT * i;
      const int grp = item % (C::TK / 4), ch = item / (C::TK / 4);
      if (item < C::TK / 4 * C::CH) {
#pragma unroll
        for (int r = 0; r < 4; ++r)
          tl.v[i][r] = vc[static_cast<int64_t>(row0 + 4 * grp + r) * C::CH + ch];
      }
    }
    return;
  }
#pragma unroll
  for (int i = 0; i < C::NKL; ++i) {
    const int item = tid + C::NT * i;
    const int key = item / C::CH, ch = item % C::CH;
    const int row = item < C::TK * C::CH ? key_row<SPARSE>(src, rows, t0, key) : -1;
    tl.k[i] = load_row_chunk(kc, row, ch, C::CH);
  }
#pragma unroll
  for (int i = 0; i < C::NVG; ++i) {
    const int item = tid + C::NT * i;
    // groups vary fastest across lanes: the transposed 8-byte LDS writes of a
    // wave then spread over a whole V^T row instead of one bank column
    const int grp = item % (C::TK / 4), ch = item / (C::TK / 4);
    const bool ok = item < C::TK / 4 * C::CH;
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const int row = ok ? key_row<SPARSE>(src, rows, t0, 4 * grp + r) : -1;
      tl.v[i][r] = load_row_chunk(vc, row, ch, C::CH);
    }
  }
}

template <class C>
__device__ __forceinline__ void store_tile(const Tile<C> &tl, char *ks, char *vt, int tid) {
#pragma unroll
  for (int i = 0; i < C::NKL; ++i) {
    const int item = tid + C::NT * i;
    if (item >= C::TK * C::CH) break;
    const int key = item / C::CH, ch = item % C::CH;
    *reinterpret_cast<uint4 *>(ks + key * C::KSTRIDE + ch * 16) = tl.k[i];
  }
#pragma unroll
  for (int i = 0; i < C::NVG; ++i) {
    const int item = tid + C::NT * i;
    if (item >= C::TK / 4 * C::CH) break;
    const int grp = item % (C::TK / 4), ch = item / (C::TK / 4);
    const int p0 = swap_bits23(4 * grp);  // 4 consecutive positions p0..p0+3
    const uint32_t *w0 = reinterpret_cast<const uint32_t *>(&tl.v[i][0]);
    const uint32_t *w1 = reinterpret_cast<const uint32_t *>(&tl.v[i][1]);
    const uint32_t *w2 = reinterpret_cast<const uint32_t *>(&tl.v[i][2]);
    const uint32_t *w3 = reinterpret_cast<const uint32_t *>(&tl.v[i][3]);
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      const int d = 8 * ch + e;
      const int w = e >> 1;
      uint2 val;
      if (e & 1) {
        val.x = pack_hi(w0[w], w1[w]);
        val.y = pack_hi(w2[w], w3[w]);
      } else {
        val.x = pack_lo(w0[w], w1[w]);
        val.y = pack_lo(w2[w], w3[w]);
      }
      *reinterpret_cast<uint2 *>(vt + d * C::VSTRIDE + p0 * 2) = val;
    }
  }
}

template <class C, bool SPARSE>
__global__ __launch_bounds__(C::NT, 1) void attn_partial_mfma(Plan P) {
  __shared__ __attribute__((aligned(16))) char smem[2][C::BUF_BYTES];
  // sparse slots: cache rows of tiles j, j+1, j+2 (ring of three)
  __shared__ int32_t srows[SPARSE ? 3 : 1][SPARSE ? C::TK : 1];

  const int tid = threadIdx.x;
  const int wave = tid / kWave, lane = tid % kWave;
  const int l32 = lane & 31, hf = lane >> 5;
  const int kg = wave % C::KG, rg = wave / C::KG;

  int bid = blockIdx.x;
  const int rc = bid % P.row_chunks;
  bid /= P.row_chunks;
  const int BH = P.B * P.Hkv;
  const int bg = bid % BH;
  const int slot = bid / BH;
  const int b = bg / P.Hkv, g = bg % P.Hkv;
  const bool tree = slot == P.tree_slot;

  // ---- the key range of this slot ----------------------------------------
  const int c = min(max(P.ctx_lens[b], 0), P.cap - P.N);
  KeySource src;
  int t_begin;
  src.c = c;
  src.idx = nullptr;
  if (tree) {
    src.off = c;
    t_begin = 0;
    src.t_end = P.N;
  } else {
    src.off = 0;
    const int lim = SPARSE ? P.n_sel : c;
    t_begin = slot * P.keys_per_split;
    src.t_end = min(t_begin + P.keys_per_split, lim);
    if (SPARSE) src.idx = P.kv_idx + static_cast<int64_t>(bg) * P.n_sel;
  }
  const int n_tiles = src.t_end > t_begin ? (src.t_end - t_begin + C::TK - 1) / C::TK : 0;

  // ---- this wave's query rows ----------------------------------------------
  const int row_base = rc * C::ROWS + rg * (C::QB * 32);
  const int part = slot * C::KG + kg;
  const int64_t prow0 = (static_cast<int64_t>(part) * BH + bg) * P.R;

  if (n_tiles == 0) {  // empty slot: (o, lse) = (0, -inf)
#pragma unroll
    for (int qb = 0; qb < C::QB; ++qb) {
      const int r = row_base + qb * 32 + l32;
      if (r < P.R && hf == 0) P.lse_part[prow0 + r] = kNegInf;
    }
    return;
  }

  const uint4 *qv = static_cast<const uint4 *>(P.q);
  bf16x8 qf[C::QB][C::DK];
  uint64_t anc_q[C::QB];
  int tree_bad = 0;
  uint64_t anc_lane = 0;
  if (tree) {
    if (P.anc == nullptr) {
      bool bad;
      anc_lane = tree_ancestors(P.parent + static_cast<int64_t>(b) * P.N, P.N, lane, &bad);
      tree_bad = bad;
    }
  }
#pragma unroll
  for (int qb = 0; qb < C::QB; ++qb) {
    const int r = row_base + qb * 32 + l32;
    const bool ok = r < P.R;
    const int i = ok ? r / P.G : 0;
    const int h = g * P.G + (ok ? r % P.G : 0);
    const int64_t qrow = (static_cast<int64_t>(b) * P.N + i) * P.Hq + h;
#pragma unroll
    for (int ks = 0; ks < C::DK; ++ks) {
      uint4 u = ok ? qv[qrow * C::CH + 2 * ks + hf] : make_uint4(0, 0, 0, 0);
      qf[qb][ks] = __builtin_bit_cast(bf16x8, u);
    }
    anc_q[qb] = 0;
    if (tree) {
      if (P.anc_words > 1)  // trees of more than 64 nodes: the row's mask words
        anc_q[qb] = reinterpret_cast<uintptr_t>(P.anc + (static_cast<int64_t>(b) * P.N + i) *
                                                           P.anc_words);
      else if (P.anc)
        anc_q[qb] = P.anc[static_cast<int64_t>(b) * P.N + i];
      else
        anc_q[qb] = shfl_u64(anc_lane, i);
    }
  }
  (void)tree_bad;

  floatx16 o_acc[C::DB][C::QB];
#pragma unroll
  for (int db = 0; db < C::DB; ++db)
#pragma unroll
    for (int qb = 0; qb < C::QB; ++qb) o_acc[db][qb] = floatx16{};
  float m_run[C::QB], l_run[C::QB];
#pragma unroll
  for (int qb = 0; qb < C::QB; ++qb) {
    m_run[qb] = kNegInf;
    l_run[qb] = 0.f;
  }

  const int64_t kv_row0 = static_cast<int64_t>(bg) * P.cap;
  const uint4 *kc = static_cast<const uint4 *>(P.k) + kv_row0 * C::CH;
  const uint4 *vc = static_cast<const uint4 *>(P.v) + kv_row0 * C::CH;
  const float cs = P.scale_log2;
  const int kbase = kg * 32 * C::KBW;

  // Row table of a sparse slot's tile (one thread per key).
  const bool gather = SPARSE && src.idx != nullptr;
  auto fill_rows = [&](int jt) -> int {
    return tid < C::TK ? index_row(src, t_begin + jt * C::TK + tid) : -1;
  };
  if (gather) {
    const int r0 = fill_rows(0), r1 = fill_rows(1);
    if (tid < C::TK) {
      srows[0][tid] = r0;
      srows[1 % (SPARSE ? 3 : 1)][tid] = r1;
    }
    __syncthreads();
  }
  const int32_t *rows0 = &srows[0][0];

  Tile<C> tl;
  load_tile<C, SPARSE>(tl, kc, vc, src, rows0, t_begin, tid);
  store_tile<C>(tl, smem[0], smem[0] + C::K_BYTES, tid);
  __syncthreads();

  for (int j = 0; j < n_tiles; ++j) {
    const int buf = j & 1;
    const int t0 = t_begin + j * C::TK;
    const bool more = j + 1 < n_tiles;
    if (more)
      load_tile<C, SPARSE>(tl, kc, vc, src, &srows[SPARSE ? (j + 1) % 3 : 0][0], t0 + C::TK,
                           tid);
    // indices of tile j+2, written to the ring after this tile's compute
    const int next_rows = gather && j + 2 < n_tiles ? fill_rows(j + 2) : -1;

    const char *ks = smem[buf];
    const char *vt = smem[buf] + C::K_BYTES;
    const int nv = min(C::TK, src.t_end - t0);

    // One 32-key block at a time: S^T = K . Q^T, online softmax, O^T += V^T . P^T.
#pragma unroll
    for (int kb = 0; kb < C::KBW; ++kb) {
      const int kb0 = kbase + 32 * kb;
      floatx16 s[C::QB];
#pragma unroll
      for (int qb = 0; qb < C::QB; ++qb) s[qb] = floatx16{};
      {
        const int key = kb0 + l32;
        const char *krow = ks + key * C::KSTRIDE + hf * 16;
#pragma unroll
        for (int kstep = 0; kstep < C::DK; ++kstep) {
          const bf16x8 a = *reinterpret_cast<const bf16x8 *>(krow + kstep * 32);
#pragma unroll
          for (int qb = 0; qb < C::QB; ++qb)
            s[qb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, qf[qb][kstep], s[qb], 0, 0, 0);
        }
      }

      // Sparse slots: a key whose index lies outside [0, c) (an out-of-range
      // entry or the -1 tail) was loaded as a zero row and takes no part.
      // The tile's row table (ring slot j % 3, not refilled before the next
      // tile) holds -1 for it; bit i of valid_w is key kb0 + i.
      uint32_t valid_w = ~0u;
      if (gather)
        valid_w = static_cast<uint32_t>(__ballot(srows[SPARSE ? j % 3 : 0][SPARSE ? kb0 + l32 : 0] >= 0));

      // mask: keys past the slot's end, invalid sparse keys and the tree's
      // non-ancestors.  The lane's 16 keys are kb0 + 4*hf + (8j + r); bit
      // 8j + r of `keep` says whether that key is visible.
      if (tree || kb0 + 32 > nv || valid_w != ~0u) {
        const int room = nv - kb0 - 4 * hf;  // visible keys start at bit 0
        uint32_t lim = room <= 0 ? 0u : room >= 32 ? ~0u : ((1u << room) - 1u);
        lim &= valid_w >> (4 * hf);
#pragma unroll
        for (int qb = 0; qb < C::QB; ++qb) {
          uint32_t keep = lim;
          if (tree) {
            // draft node of the block's first key: tile base plus block offset
            const int kt = t0 + kb0;
            const int sh = kt + 4 * hf;
            if (P.anc_words > 1) {
              // the 32-bit chunk kt / 32 of the row's mask (kt is a multiple
              // of 32 and the lane's keys lie in [kt, kt + 32)); anc_q holds
              // the address of the row's words
              const uint32_t *a32 = reinterpret_cast<const uint32_t *>(anc_q[qb]);
              const int ch = kt >> 5;
              keep &= ch < 2 * P.anc_words ? a32[ch] >> (4 * hf) : 0u;
            } else {
              keep &= sh < 64 ? static_cast<uint32_t>(anc_q[qb] >> sh) : 0u;
            }
          }
#pragma unroll
          for (int e = 0; e < 16; ++e) {
            const int bit = 8 * (e >> 2) + (e & 3);
            s[qb][e] = ((keep >> bit) & 1u) ? s[qb][e] : kNegInf;
          }
        }
      }

      // Online softmax in the log2 domain.  The running reference m_run only
      // moves when the block maximum exceeds it by more than kSlack (or on
      // the first visible key), so O is rarely rescaled; any reference gives
      // the same normalised result, and p <= 2^kSlack keeps fp32/bf16 safe.
      // P^T is packed to bf16 as the next B operand.
      bf16x8 pb[C::QB][2];
      bool rescale = false;
      float alpha[C::QB];
#pragma unroll
      for (int qb = 0; qb < C::QB; ++qb) {
        float mx = kNegInf;
#pragma unroll
        for (int e = 0; e < 16; ++e) mx = fmaxf(mx, s[qb][e]);
        mx = fmaxf(mx, __shfl_xor(mx, 32, kWave)) * cs;
        const bool move = mx > m_run[qb] + kSlack;
        const float m_new = move ? mx : m_run[qb];
        const float m_use = m_new == kNegInf ? 0.f : m_new;
        alpha[qb] = move ? fast_exp2(m_run[qb] - m_use) : 1.f;
        // nothing to rescale before the first visible key: o_acc is still 0
        rescale |= move && m_run[qb] != kNegInf;
        float sum = 0.f;
#pragma unroll
        for (int e = 0; e < 16; ++e) {
          const float p = fast_exp2(fmaf(s[qb][e], cs, -m_use));
          s[qb][e] = p;
          sum += p;
        }
#pragma unroll
        for (int half = 0; half < 2; ++half) {
          floatx8 x;
#pragma unroll
          for (int e = 0; e < 8; ++e) x[e] = s[qb][8 * half + e];
          pb[qb][half] = __builtin_convertvector(x, bf16x8);
        }
        l_run[qb] = l_run[qb] * alpha[qb] + sum;
        m_run[qb] = m_new;
      }
      if (__builtin_expect(__any(rescale), 0)) {
#pragma unroll
        for (int db = 0; db < C::DB; ++db)
#pragma unroll
          for (int qb = 0; qb < C::QB; ++qb) o_acc[db][qb] *= alpha[qb];
      }

#pragma unroll
      for (int db = 0; db < C::DB; ++db) {
        const int d = 32 * db + l32;
        const char *vrow = vt + d * C::VSTRIDE + hf * 16;
#pragma unroll
        for (int half = 0; half < 2; ++half) {
          const bf16x8 a = *reinterpret_cast<const bf16x8 *>(vrow + (kb0 + 16 * half) * 2);
#pragma unroll
          for (int qb = 0; qb < C::QB; ++qb)
            o_acc[db][qb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, pb[qb][half],
                                                                    o_acc[db][qb], 0, 0, 0);
        }
      }
    }

    if (more) store_tile<C>(tl, smem[buf ^ 1], smem[buf ^ 1] + C::K_BYTES, tid);
    if (gather && j + 2 < n_tiles && tid < C::TK) srows[SPARSE ? (j + 2) % 3 : 0][tid] = next_rows;
    __syncthreads();
  }

  // ---- epilogue: normalise, write this wave's partial -----------------------
#pragma unroll
  for (int qb = 0; qb < C::QB; ++qb) {
    const int r = row_base + qb * 32 + l32;
    const float l_tot = l_run[qb] + __shfl_xor(l_run[qb], 32, kWave);
    const float inv = l_tot > 0.f ? 1.f / l_tot : 0.f;
    if (r < P.R) {
      float *dst = P.o_part + (prow0 + r) * C::D;
#pragma unroll
      for (int db = 0; db < C::DB; ++db)
#pragma unroll
        for (int jj = 0; jj < 4; ++jj) {
          float4 v4;
          v4.x = o_acc[db][qb][4 * jj + 0] * inv;
          v4.y = o_acc[db][qb][4 * jj + 1] * inv;
          v4.z = o_acc[db][qb][4 * jj + 2] * inv;
          v4.w = o_acc[db][qb][4 * jj + 3] * inv;
          *reinterpret_cast<float4 *>(dst + 32 * db + 8 * jj + 4 * hf) = v4;
        }
      if (hf == 0)
        P.lse_part[prow0 + r] = l_tot > 0.f ? (m_run[qb] + fast_log2(l_tot)) * kLn2 : kNegInf;
    }
  }
}

template <class C>
hipError_t launch_cfg(const Plan &p, hipStream_t s) {
  const int64_t blocks = static_cast<int64_t>(p.n_slots) * p.B * p.Hkv * p.row_chunks;
  if (p.n_sel > 0)
    hipLaunchKernelGGL((attn_partial_mfma<C, true>), dim3(static_cast<unsigned>(blocks)),
                       dim3(C::NT), 0, s, p);
  else
    hipLaunchKernelGGL((attn_partial_mfma<C, false>), dim3(static_cast<unsigned>(blocks)),
                       dim3(C::NT), 0, s, p);
  return hipGetLastError();
}

// Variants: <D, waves, key-waves, 32-query blocks per wave, 32-key blocks per wave>
template <int D> using Cfg32 = Cfg<D, 4, 4, 1, 1>;   // <= 32 rows, 128-key tiles
template <int D> using Cfg64 = Cfg<D, 8, 4, 1, 1>;   // <= 64 rows, 128-key tiles
template <int D> using Cfg128 = Cfg<D, 8, 2, 1, 1>;  // <= 128 rows, 64-key tiles
template <int D> using Cfg256 = Cfg<D, 8, 1, 1, 2>;  // 256-row chunks, 64-key tiles

template <int D>
hipError_t launch_d(const Plan &p, hipStream_t s) {
  switch (p.kernel) {
    case kKernMfma32: return launch_cfg<Cfg32<D>>(p, s);
    case kKernMfma64: return launch_cfg<Cfg64<D>>(p, s);
    case kKernMfma128: return launch_cfg<Cfg128<D>>(p, s);
    default: return launch_cfg<Cfg256<D>>(p, s);
  }
}

}  // namespace

// Shape of each MFMA variant, for the host planner.
MfmaShape mfma_shape(int kernel, int head_dim) {
  (void)head_dim;
  switch (kernel) {
    case kKernMfma32: return {Cfg32<128>::KG, Cfg32<128>::TK, Cfg32<128>::ROWS};
    case kKernMfma64: return {Cfg64<128>::KG, Cfg64<128>::TK, Cfg64<128>::ROWS};
    case kKernMfma128: return {Cfg128<128>::KG, Cfg128<128>::TK, Cfg128<128>::ROWS};
    default: return {Cfg256<128>::KG, Cfg256<128>::TK, Cfg256<128>::ROWS};
  }
}

hipError_t launch_attn_partials_mfma(const Plan &p, hipStream_t s) {
  return p.D == 64 ? launch_d<64>(p, s) : launch_d<128>(p, s);
}

}  // namespace hsv
