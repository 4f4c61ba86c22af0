// Partial verification attention on the vector ALUs (fp32 arithmetic).
//
// Used for fp32 inputs and for shapes the MFMA kernel does not take.  One
// wave owns one grouped query row of one (b, kv head, part); a part is a
// contiguous range of prefix keys (LongSpec section 2.C, cache part: no
// mask) or the draft block under the ancestor mask (speculative part).
// Per 64-key chunk: lane <-> key for the scores, then lane <-> feature for
// P.V, with probabilities broadcast by v_readlane.  Both loops have fixed trip
// counts and no branches, so their loads are issued together rather than one
// memory latency at a time.  Online softmax in the log2 domain; the partial
// is stored normalised with its natural-log LSE.
#include "common.hpp"
#include "launch.h"

namespace hsv {
namespace {

constexpr int kRowsPerBlock = 4;  // one row per wave

template <int IN, int D>
__global__ __launch_bounds__(256) void attn_partial_valu(Plan P) {
  using E = Elem<IN>;
  using T = typename E::T;
  constexpr int DL = D / kWave;  // features per lane in P.V
  __shared__ float q_s[kRowsPerBlock][D];

  const int wave = threadIdx.x / kWave;
  const int lane = threadIdx.x % kWave;
  const int r = blockIdx.x * kRowsPerBlock + wave;
  const int part = blockIdx.y;
  const int bg = blockIdx.z;
  const int b = bg / P.Hkv;
  const int g = bg % P.Hkv;
  const bool active = r < P.R;
  const int i = active ? r / P.G : 0;
  const int h = g * P.G + (active ? r % P.G : 0);

  const T *q = static_cast<const T *>(P.q);
  const T *kc = static_cast<const T *>(P.k);
  const T *vc = static_cast<const T *>(P.v);

  for (int d = lane; d < D; d += kWave)
    q_s[wave][d] = active ? E::load(q, ((static_cast<int64_t>(b) * P.N + i) * P.Hq + h) * D + d)
                          : 0.f;
  __syncthreads();
  if (!active) return;

  // Out-of-contract device data must not turn into out-of-bounds reads:
  // clamp the context so the draft block stays inside the cache, and drop
  // indices outside [0, c) (the validation flag reports both).
  const int c = min(max(P.ctx_lens[b], 0), P.cap - P.N);
  const bool tree = part == P.tree_slot;
  int t_begin, t_end;
  uint64_t anc_i = 0;
  if (tree) {
    t_begin = 0;
    t_end = P.N;
    if (P.anc_words > 1) {
      anc_i = 0;  // trees of more than 64 nodes: one mask word per 64-key chunk below
    } else if (P.anc) {
      anc_i = P.anc[static_cast<int64_t>(b) * P.N + i];
    } else {
      bool bad;
      uint64_t a = tree_ancestors(P.parent + static_cast<int64_t>(b) * P.N, P.N, lane, &bad);
      anc_i = shfl_u64(a, i);
    }
  } else {
    const int limit = P.n_sel > 0 ? P.n_sel : c;
    t_begin = part * P.keys_per_split;
    t_end = min(t_begin + P.keys_per_split, limit);
  }

  const int64_t kv_base = static_cast<int64_t>(bg) * P.cap;
  const int32_t *idx = P.n_sel > 0 ? P.kv_idx + static_cast<int64_t>(bg) * P.n_sel : nullptr;

  float m = kNegInf;  // running max, log2 domain
  float l = 0.f;      // running sum of exp2(s - m)
  float acc[DL];
#pragma unroll
  for (int j = 0; j < DL; ++j) acc[j] = 0.f;

  for (int t0 = t_begin; t0 < t_end; t0 += kWave) {
    const int t = t0 + lane;
    bool valid = t < t_end;
    int pos = 0;
    if (tree) {
      pos = c + t;
      // word t0 / 64 of the row's mask (wave-uniform: t0 is a multiple of 64)
      const uint64_t word = P.anc_words > 1
                                ? P.anc[(static_cast<int64_t>(b) * P.N + i) * P.anc_words +
                                        min(t0 >> 6, P.anc_words - 1)]
                                : anc_i;
      valid = valid && ((word >> (t & 63)) & 1u);
    } else if (valid) {
      pos = idx ? idx[t] : t;
      valid = pos >= 0 && pos < c;
    }
    // keys that take no part read row 0 of the slot (in bounds) and are
    // dropped below; their values never reach the sums
    if (!valid) pos = 0;
    float s = kNegInf;
    {
      const T *krow = kc + (kv_base + pos) * D;
      float kr[D];
#pragma unroll
      for (int d = 0; d < D; ++d) kr[d] = E::load(krow, d);
      float dot = 0.f;
#pragma unroll
      for (int d = 0; d < D; ++d) dot = fmaf(q_s[wave][d], kr[d], dot);
      if (valid) s = dot * P.scale_log2;
    }
    const float m_new = fmaxf(m, wave_max(s));
    if (m_new == kNegInf) continue;
    const float alpha = fast_exp2(m - m_new);
    const float p = valid ? fast_exp2(s - m_new) : 0.f;
    l = l * alpha + wave_sum(p);
#pragma unroll
    for (int j = 0; j < DL; ++j) acc[j] *= alpha;
    // every lane of the chunk in turn (p = 0 past the range and for dropped
    // keys): a zero weight selects 0 instead of the row's value, so a
    // non-finite entry of a row that takes no part cannot reach acc
#pragma unroll 16
    for (int jj = 0; jj < kWave; ++jj) {
      const float pj = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(p), jj));
      const int posj = __builtin_amdgcn_readlane(pos, jj);
      const T *vrow = vc + (kv_base + posj) * D;
#pragma unroll
      for (int j = 0; j < DL; ++j) {
        const float x = E::load(vrow, lane + j * kWave);
        acc[j] = fmaf(pj, pj != 0.f ? x : 0.f, acc[j]);
      }
    }
    m = m_new;
  }

  const int64_t prow = (static_cast<int64_t>(part) * P.B * P.Hkv + bg) * P.R + r;
  const float inv = l > 0.f ? 1.f / l : 0.f;
#pragma unroll
  for (int j = 0; j < DL; ++j) P.o_part[prow * D + lane + j * kWave] = acc[j] * inv;
  if (lane == 0) P.lse_part[prow] = l > 0.f ? (m + fast_log2(l)) * kLn2 : kNegInf;
}

template <int IN, int D>
hipError_t launch_valu(const Plan &p, hipStream_t s) {
  dim3 grid((p.R + kRowsPerBlock - 1) / kRowsPerBlock, p.n_parts, p.B * p.Hkv);
  hipLaunchKernelGGL((attn_partial_valu<IN, D>), grid, dim3(256), 0, s, p);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_attn_partials_valu(const Plan &p, hipStream_t s) {
  if (p.in_dtype == kF32) return p.D == 64 ? launch_valu<kF32, 64>(p, s) : launch_valu<kF32, 128>(p, s);
  return p.D == 64 ? launch_valu<kBF16, 64>(p, s) : launch_valu<kBF16, 128>(p, s);
}

}  // namespace hsv
