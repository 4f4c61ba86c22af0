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

// --------------------------------------------------------------------------
// Log-sum-exp merge (LongSpec section 2.C: exact combination of the parts).
// One wave per output row; lane l owns features 2l, 2l+1 (D = 128) or l
// (D = 64).  Lane p reads part p's LSE, the wave reduces them to
// lse = m + log sum exp(lse_p - m), and the per-part weights exp(lse_p - lse)
// are broadcast with v_readlane while eight parts' rows are in flight.
// Parts with lse = -inf get weight 0 and their (possibly never written) o
// rows are discarded by a select, so they cannot inject NaN.
// --------------------------------------------------------------------------
constexpr int kMergeRowsPerBlock = 4;  // 256 threads, one wave per row

template <int D>
__device__ __forceinline__ void merge_row(const float *o_parts, const float *lse_parts,
                                          int n_parts, int64_t part_stride_rows, int64_t row,
                                          int lane, float (&acc)[D / 64], float *lse_out) {
  constexpr int DL = D / 64;
  const float *lp = lse_parts + row;
  float m = kNegInf;
  for (int p = lane; p < n_parts; p += kWave) m = fmaxf(m, lp[p * part_stride_rows]);
  m = wave_max(m);
#pragma unroll
  for (int j = 0; j < DL; ++j) acc[j] = 0.f;
  if (m == kNegInf) {
    *lse_out = kNegInf;
    return;
  }
  float sum = 0.f;
  for (int p = lane; p < n_parts; p += kWave)
    sum += fast_exp2((lp[p * part_stride_rows] - m) * kLog2e);
  sum = wave_sum(sum);
  const float lse = m + fast_log2(sum) * kLn2;
  const float *op = o_parts + row * D + lane * DL;
  const int64_t ostride = part_stride_rows * D;
  constexpr int kBatch = 8;
  for (int p0 = 0; p0 < n_parts; p0 += kWave) {
    const int p = p0 + lane;
    const float w_lane = p < n_parts ? fast_exp2((lp[p * part_stride_rows] - lse) * kLog2e) : 0.f;
    const int n_here = min(kWave, n_parts - p0);
    for (int u0 = 0; u0 < n_here; u0 += kBatch) {
      float w[kBatch];
      float v[kBatch][DL];
#pragma unroll
      for (int u = 0; u < kBatch; ++u) {
        const int q = min(p0 + u0 + u, n_parts - 1);  // stays in bounds
        w[u] = u0 + u < n_here
                   ? __int_as_float(__builtin_amdgcn_readlane(__float_as_int(w_lane), u0 + u))
                   : 0.f;
#pragma unroll
        for (int j = 0; j < DL; ++j) v[u][j] = op[q * ostride + j];
      }
#pragma unroll
      for (int u = 0; u < kBatch; ++u)
#pragma unroll
        for (int j = 0; j < DL; ++j) acc[j] = fmaf(w[u], w[u] != 0.f ? v[u][j] : 0.f, acc[j]);
    }
  }
  *lse_out = lse;
}

template <int D>
__device__ __forceinline__ void store_row(void *o, int out_dtype, int64_t base,
                                          const float (&acc)[D / 64], int lane) {
  constexpr int DL = D / 64;
  if (out_dtype == kF32) {
    float *dst = static_cast<float *>(o) + base + lane * DL;
#pragma unroll
    for (int j = 0; j < DL; ++j) dst[j] = acc[j];
  } else {
    uint16_t *dst = static_cast<uint16_t *>(o) + base + lane * DL;
#pragma unroll
    for (int j = 0; j < DL; ++j) dst[j] = f32_to_bf16_rne(acc[j]);
  }
}

template <int D>
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
  float acc[D / 64];
  float lse;
  merge_row<D>(P.o_part, P.lse_part, P.n_parts, stride, prow, lane, acc, &lse);
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
  float acc[D / 64];
  float l;
  merge_row<D>(o_parts, lse_parts, n_parts, n_rows, row, lane, acc, &l);
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
      const int t = row[s];
      if (t < 0 || t >= c || (s > 0 && row[s - 1] >= t)) bits |= kErrIndex;
    }
  }
  if (bits) atomicOr(P.err, bits);
}

}  // namespace

hipError_t launch_tree_mask(const int32_t *parent, uint64_t *anc, int batch, int n_draft,
                            hipStream_t s) {
  hipLaunchKernelGGL(tree_mask_kernel, dim3(batch), dim3(64), 0, s, parent, anc, n_draft);
  return hipGetLastError();
}

hipError_t launch_merge_verify(const Plan &p, hipStream_t s) {
  const int64_t rows = static_cast<int64_t>(p.B) * p.N * p.Hq;
  dim3 grid(static_cast<unsigned>((rows + kMergeRowsPerBlock - 1) / kMergeRowsPerBlock));
  if (p.D == 64)
    hipLaunchKernelGGL(merge_verify_kernel<64>, grid, dim3(256), 0, s, p);
  else
    hipLaunchKernelGGL(merge_verify_kernel<128>, grid, dim3(256), 0, s, p);
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
