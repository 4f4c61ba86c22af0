// Small kernels around the attention partials: the ancestor bitmask, the
// log-sum-exp merge, the sparse-cache gather and the precondition check.
#include "common.hpp"
#include "launch.h"

namespace hsv {
namespace {

// --------------------------------------------------------------------------
// Ancestor bitmask (LongSpec section 2.C, the tree-branch mask): one wave per
// sequence, lane i = draft node i, pointer jumping with 64-bit shuffles.
// --------------------------------------------------------------------------
__global__ __launch_bounds__(64) void tree_mask_kernel(const int32_t *parent, uint64_t *anc,
                                                       int n_draft) {
  const int b = blockIdx.x;
  const int lane = threadIdx.x;
  bool bad;
  const uint64_t a = tree_ancestors(parent + static_cast<int64_t>(b) * n_draft, n_draft, lane,
                                    &bad);
  if (lane < n_draft) anc[static_cast<int64_t>(b) * n_draft + lane] = bad ? 0 : a;
}

// Ancestor bitmask of trees of 65 to 256 nodes: W = ceil(N/64) words per
// node, word w holding nodes 64w .. 64w+63.  One 256-thread workgroup per
// sequence; thread i walks its parent chain (parents in LDS; a valid array
// strictly decreases along it, so at most i steps) into four word registers.
// Every word of a sequence with an out-of-range parent is 0.
__global__ __launch_bounds__(256) void tree_mask_wide_kernel(const int32_t *parent, uint64_t *anc,
                                                             int n_draft) {
  __shared__ int32_t par[256];
  __shared__ int32_t bad;
  const int b = blockIdx.x, i = threadIdx.x;
  if (i == 0) bad = 0;
  __syncthreads();
  if (i < n_draft) {
    const int p = parent[static_cast<int64_t>(b) * n_draft + i];
    par[i] = p;
    if (p < -1 || p >= i) atomicOr(&bad, 1);
  }
  __syncthreads();
  if (i >= n_draft) return;
  uint64_t w0 = 0, w1 = 0, w2 = 0, w3 = 0;
  if (!bad) {
    for (int j = i; j >= 0; j = par[j]) {
      const uint64_t bit = uint64_t{1} << (j & 63);
      const int wi = j >> 6;
      w0 |= wi == 0 ? bit : 0;
      w1 |= wi == 1 ? bit : 0;
      w2 |= wi == 2 ? bit : 0;
      w3 |= wi == 3 ? bit : 0;
    }
  }
  const int W = (n_draft + 63) / 64;
  uint64_t *row = anc + (static_cast<int64_t>(b) * n_draft + i) * W;
  row[0] = w0;
  if (W > 1) row[1] = w1;
  if (W > 2) row[2] = w2;
  if (W > 3) row[3] = w3;
}

// --------------------------------------------------------------------------
// Log-sum-exp merge (LongSpec section 2.C: exact combination of the parts).
// One wave per output row.  A part's row of D floats is read by L = D/4
// lanes (16 bytes each), so one load instruction covers S = 64/L parts;
// lane l takes sub-group l / L and features 4*(l % L) .. +3.  All loads of a
// group of 32 parts (and the LSE of every part) are issued before any is
// used, so a row costs about one memory latency instead of one per batch.
// lse = m + log sum_p exp(lse_p - m); O = sum_p exp(lse_p - lse) * O_p.
// Parts with lse = -inf get weight 0 and their (possibly never written) rows
// are discarded by a select, so they cannot inject NaN.  The S sub-group
// sums are combined with cross-lane adds; lanes of sub-group 0 end up with
// the row.  With F16 the part rows are fp16, each to be multiplied by its
// power-of-two scale (o_scale), which is folded into the part's weight.
// --------------------------------------------------------------------------
constexpr int kMergeRowsPerBlock = 4;  // 256 threads, one wave per row
constexpr int kMergeGroup = 32;        // parts whose rows are in flight together

typedef _Float16 halfx4 __attribute__((ext_vector_type(4)));

template <bool F16>
__device__ __forceinline__ float4 load4(const void *base, int64_t elem) {
  if constexpr (F16) {
    const halfx4 h = *reinterpret_cast<const halfx4 *>(static_cast<const _Float16 *>(base) + elem);
    return make_float4(static_cast<float>(h[0]), static_cast<float>(h[1]),
                       static_cast<float>(h[2]), static_cast<float>(h[3]));
  } else {
    return *reinterpret_cast<const float4 *>(static_cast<const float *>(base) + elem);
  }
}

template <int D, bool F16>
__device__ __forceinline__ void merge_row(const void *o_parts, const float *lse_parts,
                                          const float *o_scale, int n_parts,
                                          int64_t part_stride_rows, int64_t row, int lane,
                                          float4 *acc_out, float *lse_out) {
  constexpr int L = D / 4;           // lanes per part row
  constexpr int S = kWave / L;       // parts per load instruction
  constexpr int U = kMergeGroup / S; // loads per lane per group
  const int sub = lane / L, c = lane % L;
  const float *lp = lse_parts + row;
  const float *sp = F16 ? o_scale + row : nullptr;
  const int64_t o0 = row * D + 4 * c;
  const int64_t ostride = part_stride_rows * D;

  // first group's rows: in flight with the LSE loads
  float4 v[U];
#pragma unroll
  for (int u = 0; u < U; ++u) {
    const int p = min(S * u + sub, n_parts - 1);  // stays in bounds
    v[u] = load4<F16>(o_parts, o0 + p * ostride);
  }
  // LSEs (and row scales): parts 0..63 in flight with the rows, the rest (if
  // any) by a loop
  const float l0 = lane < n_parts ? lp[static_cast<int64_t>(lane) * part_stride_rows] : kNegInf;
  const float s0 =
      (F16 && lane < n_parts) ? sp[static_cast<int64_t>(lane) * part_stride_rows] : 0.f;
  float m = l0;
  for (int p = lane + kWave; p < n_parts; p += kWave) m = fmaxf(m, lp[p * part_stride_rows]);
  m = wave_max(m);
  float4 acc = make_float4(0.f, 0.f, 0.f, 0.f);
  if (m == kNegInf) {
    *acc_out = acc;
    *lse_out = kNegInf;
    return;
  }
  float sum = fast_exp2((l0 - m) * kLog2e);  // -inf -> 0
  for (int p = lane + kWave; p < n_parts; p += kWave)
    sum += fast_exp2((lp[p * part_stride_rows] - m) * kLog2e);
  sum = wave_sum(sum);
  const float lse = m + fast_log2(sum) * kLn2;

  for (int p0 = 0; p0 < n_parts; p0 += kMergeGroup) {
    if (p0 > 0) {
#pragma unroll
      for (int u = 0; u < U; ++u) {
        const int p = min(p0 + S * u + sub, n_parts - 1);
        v[u] = load4<F16>(o_parts, o0 + p * ostride);
      }
    }
    // the LSE (and scale) of part p0 + j sits in lane base + j
    float lsrc = l0, ssrc = s0;
    int base = p0;
    if (p0 >= kWave) {
      const int psrc = p0 + (lane & (kMergeGroup - 1));
      lsrc = psrc < n_parts ? lp[psrc * part_stride_rows] : kNegInf;
      if constexpr (F16) ssrc = sp[min(psrc, n_parts - 1) * part_stride_rows];
      base = 0;
    }
    float wsrc = fast_exp2((lsrc - lse) * kLog2e);
    if constexpr (F16) wsrc = lsrc > kNegInf ? wsrc * ssrc : 0.f;
#pragma unroll
    for (int u = 0; u < U; ++u) {
      float w = 0.f;
#pragma unroll
      for (int q = 0; q < S; ++q) {
        const float wq = __int_as_float(
            __builtin_amdgcn_readlane(__float_as_int(wsrc), base + S * u + q));
        w = sub == q ? wq : w;
      }
      const bool live = p0 + S * u + sub < n_parts && w != 0.f;
      w = live ? w : 0.f;
      acc.x = fmaf(w, live ? v[u].x : 0.f, acc.x);
      acc.y = fmaf(w, live ? v[u].y : 0.f, acc.y);
      acc.z = fmaf(w, live ? v[u].z : 0.f, acc.z);
      acc.w = fmaf(w, live ? v[u].w : 0.f, acc.w);
    }
  }
#pragma unroll
  for (int off = L; off < kWave; off <<= 1) {
    acc.x += __shfl_xor(acc.x, off, kWave);
    acc.y += __shfl_xor(acc.y, off, kWave);
    acc.z += __shfl_xor(acc.z, off, kWave);
    acc.w += __shfl_xor(acc.w, off, kWave);
  }
  *acc_out = acc;
  *lse_out = lse;
}

// Lanes of sub-group 0 (lane < D/4) write features 4*lane .. 4*lane+3.
template <int D>
__device__ __forceinline__ void store_row(void *o, int out_dtype, int64_t base, float4 acc,
                                          int lane) {
  if (lane >= D / 4) return;
  if (out_dtype == kF32) {
    *reinterpret_cast<float4 *>(static_cast<float *>(o) + base + 4 * lane) = acc;
  } else {
    const uint32_t lo = f32_to_bf16_rne(acc.x) | (static_cast<uint32_t>(f32_to_bf16_rne(acc.y)) << 16);
    const uint32_t hi = f32_to_bf16_rne(acc.z) | (static_cast<uint32_t>(f32_to_bf16_rne(acc.w)) << 16);
    *reinterpret_cast<uint2 *>(static_cast<uint16_t *>(o) + base + 4 * lane) = make_uint2(lo, hi);
  }
}

template <int D, bool F16>
__global__ __launch_bounds__(256) void merge_verify_kernel(Plan P) {
  const int lane = threadIdx.x % kWave;
  const int64_t row = static_cast<int64_t>(blockIdx.x) * kMergeRowsPerBlock + threadIdx.x / kWave;
  const int64_t total = static_cast<int64_t>(P.B) * P.N * P.Hq;
  if (row >= total) return;
  const int h = static_cast<int>(row % P.Hq);
  const int i = static_cast<int>((row / P.Hq) % P.N);
  const int b = static_cast<int>(row / (static_cast<int64_t>(P.Hq) * P.N));
  const int g = h / P.G;
  const int r = i * P.G + (h % P.G);
  const int64_t prow = (static_cast<int64_t>(b) * P.Hkv + g) * P.R + r;
  const int64_t stride = static_cast<int64_t>(P.B) * P.Hkv * P.R;
  float4 acc = make_float4(0.f, 0.f, 0.f, 0.f);
  float lse = kNegInf;
  // A plan with no partials (an empty key set: no prefix keys and no tree
  // part) has nothing to read: every row is the empty-set result.
  if (P.n_parts > 0)
    merge_row<D, F16>(P.o_part, P.lse_part, P.o_scale, P.n_parts, stride, prow, lane, &acc,
                      &lse);
  store_row<D>(P.o, P.out_dtype, row * D, acc, lane);
  if (lane == 0) P.lse[row] = lse;
}

template <int D>
__global__ __launch_bounds__(256) void merge_rows_kernel(const float *o_parts,
                                                         const float *lse_parts, int n_parts,
                                                         int64_t n_rows, void *o, float *lse,
                                                         int out_dtype) {
  const int lane = threadIdx.x % kWave;
  const int64_t row = static_cast<int64_t>(blockIdx.x) * kMergeRowsPerBlock + threadIdx.x / kWave;
  if (row >= n_rows) return;
  float4 acc;
  float l;
  merge_row<D, false>(o_parts, lse_parts, nullptr, n_parts, n_rows, row, lane, &acc, &l);
  store_row<D>(o, out_dtype, row * D, acc, lane);
  if (lane == 0) lse[row] = l;
}

// --------------------------------------------------------------------------
// Compressed cache (Dustin page, verification workflow step 3): copy the
// selected rows, 16 bytes per lane.  Indices outside [0, cap) give zero rows.
// --------------------------------------------------------------------------
__global__ __launch_bounds__(256) void gather_kv_kernel(const uint4 *k, const uint4 *v,
                                                        const int32_t *idx, uint4 *k_out,
                                                        uint4 *v_out, int hkv, int cap,
                                                        int row_vec, int n_sel) {
  const int bg = blockIdx.y;
  const int64_t e = static_cast<int64_t>(blockIdx.x) * blockDim.x + threadIdx.x;
  const int64_t total = static_cast<int64_t>(n_sel) * row_vec;
  if (e >= total) return;
  const int s = static_cast<int>(e / row_vec);
  const int c = static_cast<int>(e % row_vec);
  const int t = idx[static_cast<int64_t>(bg) * n_sel + s];
  const int64_t dst = (static_cast<int64_t>(bg) * n_sel + s) * row_vec + c;
  if (t < 0 || t >= cap) {
    k_out[dst] = make_uint4(0, 0, 0, 0);
    v_out[dst] = make_uint4(0, 0, 0, 0);
    return;
  }
  const int64_t src = (static_cast<int64_t>(bg) * cap + t) * row_vec + c;
  k_out[dst] = k[src];
  v_out[dst] = v[src];
  (void)hkv;
}

// --------------------------------------------------------------------------
// Precondition check for HSV_FLAG_VALIDATE: one block per sequence.
// --------------------------------------------------------------------------
__global__ __launch_bounds__(256) void validate_kernel(Plan P) {
  const int b = blockIdx.x;
  const int c = P.ctx_lens[b];
  int32_t bits = 0;
  if (threadIdx.x == 0 && (c < 0 || c > P.max_ctx || static_cast<int64_t>(c) + P.N > P.cap))
    bits |= kErrCtx;
  if (P.parent && P.has_tree)
    for (int i = threadIdx.x; i < P.N; i += blockDim.x) {
      const int p = P.parent[static_cast<int64_t>(b) * P.N + i];
      if (p < -1 || p >= i) bits |= kErrParent;
    }
  if (P.n_sel > 0 && P.n_splits > 0) {
    const int64_t n = static_cast<int64_t>(P.Hkv) * P.n_sel;
    for (int64_t e = threadIdx.x; e < n; e += blockDim.x) {
      const int s = static_cast<int>(e % P.n_sel);
      const int32_t *row = P.kv_idx + static_cast<int64_t>(b) * n + (e - s);
      // a strictly increasing run of positions in [0, c), then -1 slots
      const int t = row[s];
      if (t != -1 && (t < 0 || t >= c || (s > 0 && (row[s - 1] >= t || row[s - 1] == -1))))
        bits |= kErrIndex;
    }
  }
  if (P.block_table && c >= 0 && static_cast<int64_t>(c) + P.N <= P.cap) {
    const int nb = (c + P.N + (1 << P.block_shift) - 1) >> P.block_shift;
    for (int j = threadIdx.x; j < nb; j += blockDim.x) {
      const int e = P.block_table[static_cast<int64_t>(b) * P.max_blocks + j];
      if (e < 0 || e >= P.n_pool_blocks) bits |= kErrIndex;
    }
  }
  if (bits) atomicOr(P.err, bits);
}

}  // namespace

hipError_t launch_tree_mask(const int32_t *parent, uint64_t *anc, int batch, int n_draft,
                            hipStream_t s) {
  if (n_draft > 64)
    hipLaunchKernelGGL(tree_mask_wide_kernel, dim3(batch), dim3(256), 0, s, parent, anc, n_draft);
  else
    hipLaunchKernelGGL(tree_mask_kernel, dim3(batch), dim3(64), 0, s, parent, anc, n_draft);
  return hipGetLastError();
}

hipError_t launch_merge_verify(const Plan &p, hipStream_t s) {
  const int64_t rows = static_cast<int64_t>(p.B) * p.N * p.Hq;
  dim3 grid(static_cast<unsigned>((rows + kMergeRowsPerBlock - 1) / kMergeRowsPerBlock));
  if (p.D == 64) {
    if (p.part_f16)
      hipLaunchKernelGGL((merge_verify_kernel<64, true>), grid, dim3(256), 0, s, p);
    else
      hipLaunchKernelGGL((merge_verify_kernel<64, false>), grid, dim3(256), 0, s, p);
  } else {
    if (p.part_f16)
      hipLaunchKernelGGL((merge_verify_kernel<128, true>), grid, dim3(256), 0, s, p);
    else
      hipLaunchKernelGGL((merge_verify_kernel<128, false>), grid, dim3(256), 0, s, p);
  }
  return hipGetLastError();
}

hipError_t launch_merge_rows(const float *o_parts, const float *lse_parts, int n_parts,
                             int64_t n_rows, int head_dim, void *o, float *lse, int out_dtype,
                             hipStream_t s) {
  dim3 grid(static_cast<unsigned>((n_rows + kMergeRowsPerBlock - 1) / kMergeRowsPerBlock));
  if (head_dim == 64)
    hipLaunchKernelGGL(merge_rows_kernel<64>, grid, dim3(256), 0, s, o_parts, lse_parts,
                       n_parts, n_rows, o, lse, out_dtype);
  else
    hipLaunchKernelGGL(merge_rows_kernel<128>, grid, dim3(256), 0, s, o_parts, lse_parts,
                       n_parts, n_rows, o, lse, out_dtype);
  return hipGetLastError();
}

hipError_t launch_gather_kv(const void *k, const void *v, const int32_t *idx, void *k_out,
                            void *v_out, int batch, int hkv, int cap, int head_dim, int n_sel,
                            int elem_bytes, hipStream_t s) {
  const int row_vec = head_dim * elem_bytes / 16;
  const int64_t total = static_cast<int64_t>(n_sel) * row_vec;
  dim3 grid(static_cast<unsigned>((total + 255) / 256), batch * hkv);
  hipLaunchKernelGGL(gather_kv_kernel, grid, dim3(256), 0, s, static_cast<const uint4 *>(k),
                     static_cast<const uint4 *>(v), idx, static_cast<uint4 *>(k_out),
                     static_cast<uint4 *>(v_out), hkv, cap, row_vec, n_sel);
  return hipGetLastError();
}

hipError_t launch_validate(const Plan &p, hipStream_t s) {
  hipLaunchKernelGGL(validate_kernel, dim3(p.B), dim3(256), 0, s, p);
  return hipGetLastError();
}

}  // namespace hsv
