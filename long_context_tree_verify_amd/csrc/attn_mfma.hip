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
// K rows and V^T rows are XOR-swizzled in 16-byte chunks against bank
// conflicts.  Waves are arranged as RG row groups x KG key groups; each wave
// writes its own partial (KG partials per slot), merged later with the rest.
#include "common.hpp"
#include "launch.h"

namespace hsv {
namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float floatx16 __attribute__((ext_vector_type(16)));
typedef float floatx8 __attribute__((ext_vector_type(8)));

template <int D_, int KG_, int QB_, int KBW_>
struct Cfg {
  static constexpr int D = D_;
  static constexpr int KG = KG_;             // waves along keys
  static constexpr int RG = 4 / KG_;         // waves along rows
  static constexpr int QB = QB_;             // 32-query blocks per wave
  static constexpr int KBW = KBW_;           // 32-key blocks per wave per tile
  static constexpr int TK = 32 * KBW * KG;   // keys per tile
  static constexpr int ROWS = RG * QB * 32;  // grouped rows per workgroup
  static constexpr int CH = D / 8;           // 16-byte chunks per K/V row
  static constexpr int DK = D / 16;          // MFMA k-steps over the features
  static constexpr int DB = D / 32;          // 32-feature blocks of O
  static constexpr int TILE_BYTES = TK * D * 2;          // K or V tile (bf16)
  static constexpr int NKL = (TK * CH + 255) / 256;      // K loads per thread
  static constexpr int NVG = (TK / 4 * CH + 255) / 256;  // 4-key V groups per thread
};

__device__ __forceinline__ int swap_bits23(int k) {
  return (k & ~12) | ((k & 4) << 1) | ((k & 8) >> 1);
}

// XOR swizzle of a V^T row's 16-byte chunks: 8 consecutive feature rows read
// the same logical chunk from 8 different banks.
__device__ __forceinline__ int vt_swizzle(int d) { return (d ^ (d >> 3)) & 7; }

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

// Where key t of this slot lives in the cache, and whether it exists.
struct KeySource {
  int mode;        // 0 dense prefix, 1 sparse prefix, 2 tree
  int c;           // context length (clamped)
  int t_end;       // keys [.., t_end) of this slot are valid
  const int32_t *idx;
  __device__ __forceinline__ int pos(int t, bool &valid) const {
    valid = t < t_end;
    if (!valid) return 0;
    if (mode == 0) return t;
    if (mode == 2) return c + t;
    const int p = idx[t];
    valid = p >= 0 && p < c;
    return valid ? p : 0;
  }
};

template <class C>
__device__ __forceinline__ void load_tile(Tile<C> &tl, const uint4 *kc, const uint4 *vc,
                                          int64_t kv_row0, const KeySource &src, int t0,
                                          int tid) {
#pragma unroll
  for (int i = 0; i < C::NKL; ++i) {
    const int item = tid + 256 * i;
    const int key = item / C::CH, ch = item % C::CH;
    bool ok = item < C::TK * C::CH;
    bool valid = false;
    const int p = ok ? src.pos(t0 + key, valid) : 0;
    tl.k[i] = valid ? kc[(kv_row0 + p) * C::CH + ch] : make_uint4(0, 0, 0, 0);
  }
#pragma unroll
  for (int i = 0; i < C::NVG; ++i) {
    const int item = tid + 256 * i;
    const int grp = item / C::CH, ch = item % C::CH;
    const bool ok = item < C::TK / 4 * C::CH;
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      bool valid = false;
      const int p = ok ? src.pos(t0 + 4 * grp + r, valid) : 0;
      tl.v[i][r] = valid ? vc[(kv_row0 + p) * C::CH + ch] : make_uint4(0, 0, 0, 0);
    }
  }
}

template <class C>
__device__ __forceinline__ void store_tile(const Tile<C> &tl, char *ks, char *vt, int tid) {
#pragma unroll
  for (int i = 0; i < C::NKL; ++i) {
    const int item = tid + 256 * i;
    if (item >= C::TK * C::CH) break;
    const int key = item / C::CH, ch = item % C::CH;
    *reinterpret_cast<uint4 *>(ks + key * C::CH * 16 + ((ch ^ (key & 7)) * 16)) = tl.k[i];
  }
#pragma unroll
  for (int i = 0; i < C::NVG; ++i) {
    const int item = tid + 256 * i;
    if (item >= C::TK / 4 * C::CH) break;
    const int grp = item / C::CH, ch = item % C::CH;
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
      char *row = vt + d * (C::TK * 2);
      *reinterpret_cast<uint2 *>(row + (((p0 >> 3) ^ vt_swizzle(d)) * 16) + (p0 & 7) * 2) = val;
    }
  }
}

template <class C>
__global__ __launch_bounds__(256, 1) void attn_partial_mfma(Plan P) {
  __shared__ __attribute__((aligned(16))) char smem[2][2 * C::TILE_BYTES];

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
  if (tree) {
    src.mode = 2;
    t_begin = 0;
    src.t_end = P.N;
  } else {
    src.mode = P.n_sel > 0 ? 1 : 0;
    const int lim = P.n_sel > 0 ? P.n_sel : c;
    t_begin = slot * P.keys_per_split;
    src.t_end = min(t_begin + P.keys_per_split, lim);
  }
  src.c = c;
  src.idx = P.n_sel > 0 ? P.kv_idx + static_cast<int64_t>(bg) * P.n_sel : nullptr;
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
      if (P.anc)
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

  const uint4 *kc = static_cast<const uint4 *>(P.k);
  const uint4 *vc = static_cast<const uint4 *>(P.v);
  const int64_t kv_row0 = static_cast<int64_t>(bg) * P.cap;
  const float cs = P.scale_log2;
  const int kbase = kg * 32 * C::KBW;

  Tile<C> tl;
  load_tile<C>(tl, kc, vc, kv_row0, src, t_begin, tid);
  store_tile<C>(tl, smem[0], smem[0] + C::TILE_BYTES, tid);
  __syncthreads();

  for (int j = 0; j < n_tiles; ++j) {
    const int buf = j & 1;
    const int t0 = t_begin + j * C::TK;
    const bool more = j + 1 < n_tiles;
    if (more) load_tile<C>(tl, kc, vc, kv_row0, src, t0 + C::TK, tid);

    const char *ks = smem[buf];
    const char *vt = smem[buf] + C::TILE_BYTES;
    const int nv = min(C::TK, src.t_end - t0);

    // S^T = K . Q^T
    floatx16 s[C::KBW][C::QB];
#pragma unroll
    for (int kb = 0; kb < C::KBW; ++kb)
#pragma unroll
      for (int qb = 0; qb < C::QB; ++qb) s[kb][qb] = floatx16{};
#pragma unroll
    for (int kstep = 0; kstep < C::DK; ++kstep) {
      bf16x8 a[C::KBW];
#pragma unroll
      for (int kb = 0; kb < C::KBW; ++kb) {
        const int key = kbase + 32 * kb + l32;
        const int chunk = 2 * kstep + hf;
        a[kb] = *reinterpret_cast<const bf16x8 *>(ks + key * C::CH * 16 +
                                                  ((chunk ^ (key & 7)) * 16));
      }
#pragma unroll
      for (int kb = 0; kb < C::KBW; ++kb)
#pragma unroll
        for (int qb = 0; qb < C::QB; ++qb)
          s[kb][qb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a[kb], qf[qb][kstep], s[kb][qb],
                                                               0, 0, 0);
    }

    // mask: keys past the slot's end, and the tree's non-ancestors
    if (tree || nv < C::TK) {
#pragma unroll
      for (int kb = 0; kb < C::KBW; ++kb)
#pragma unroll
        for (int qb = 0; qb < C::QB; ++qb)
#pragma unroll
          for (int e = 0; e < 16; ++e) {
            const int key = kbase + 32 * kb + 8 * (e >> 2) + 4 * hf + (e & 3);
            bool ok = key < nv;
            if (tree) ok = ok && ((anc_q[qb] >> (key & 63)) & 1u);
            if (!ok) s[kb][qb][e] = kNegInf;
          }
    }

    // online softmax (log2 domain), P^T packed to bf16 as the next B operand
    bf16x8 pb[C::KBW][C::QB][2];
    bool rescale = false;
    float alpha[C::QB];
#pragma unroll
    for (int qb = 0; qb < C::QB; ++qb) {
      float mx = kNegInf;
#pragma unroll
      for (int kb = 0; kb < C::KBW; ++kb)
#pragma unroll
        for (int e = 0; e < 16; ++e) mx = fmaxf(mx, s[kb][qb][e]);
      mx = fmaxf(mx, __shfl_xor(mx, 32, kWave));
      const float m_new = fmaxf(m_run[qb], mx * cs);
      const float m_use = m_new == kNegInf ? 0.f : m_new;
      alpha[qb] = fast_exp2(m_run[qb] - m_use);
      rescale |= alpha[qb] != 1.f;
      float sum = 0.f;
#pragma unroll
      for (int kb = 0; kb < C::KBW; ++kb) {
#pragma unroll
        for (int e = 0; e < 16; ++e) {
          const float p = fast_exp2(fmaf(s[kb][qb][e], cs, -m_use));
          s[kb][qb][e] = p;
          sum += p;
        }
#pragma unroll
        for (int half = 0; half < 2; ++half) {
          floatx8 x;
#pragma unroll
          for (int e = 0; e < 8; ++e) x[e] = s[kb][qb][8 * half + e];
          pb[kb][qb][half] = __builtin_convertvector(x, bf16x8);
        }
      }
      l_run[qb] = l_run[qb] * alpha[qb] + sum;
      m_run[qb] = m_new;
    }
    if (__any(rescale)) {
#pragma unroll
      for (int db = 0; db < C::DB; ++db)
#pragma unroll
        for (int qb = 0; qb < C::QB; ++qb) o_acc[db][qb] *= alpha[qb];
    }

    // O^T += V^T . P^T
#pragma unroll
    for (int db = 0; db < C::DB; ++db) {
      const int d = 32 * db + l32;
      const char *vrow = vt + d * (C::TK * 2);
      const int sw = vt_swizzle(d);
#pragma unroll
      for (int kb = 0; kb < C::KBW; ++kb)
#pragma unroll
        for (int half = 0; half < 2; ++half) {
          const int pos = kbase + 32 * kb + 16 * half + 8 * hf;
          const bf16x8 a = *reinterpret_cast<const bf16x8 *>(vrow + (((pos >> 3) ^ sw) * 16));
#pragma unroll
          for (int qb = 0; qb < C::QB; ++qb)
            o_acc[db][qb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, pb[kb][qb][half],
                                                                    o_acc[db][qb], 0, 0, 0);
        }
    }

    if (more) store_tile<C>(tl, smem[buf ^ 1], smem[buf ^ 1] + C::TILE_BYTES, tid);
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
  hipLaunchKernelGGL(attn_partial_mfma<C>, dim3(static_cast<unsigned>(blocks)), dim3(256), 0, s,
                     p);
  return hipGetLastError();
}

template <int D>
hipError_t launch_d(const Plan &p, hipStream_t s) {
  switch (p.kernel) {
    case kKernMfma32: return launch_cfg<Cfg<D, 4, 1, 1>>(p, s);
    case kKernMfma64: return launch_cfg<Cfg<D, 4, 2, 1>>(p, s);
    case kKernMfma128: return launch_cfg<Cfg<D, 2, 2, 1>>(p, s);
    default: return launch_cfg<Cfg<D, 1, 2, 2>>(p, s);
  }
}

}  // namespace

// Shape of each MFMA variant, for the host planner.
MfmaShape mfma_shape(int kernel, int head_dim) {
  (void)head_dim;
  switch (kernel) {
    case kKernMfma32: return {4, 128, 32};
    case kKernMfma64: return {4, 128, 64};
    case kKernMfma128: return {2, 64, 128};
    default: return {1, 64, 256};
  }
}

hipError_t launch_attn_partials_mfma(const Plan &p, hipStream_t s) {
  return p.D == 64 ? launch_d<64>(p, s) : launch_d<128>(p, s);
}

}  // namespace hsv
