// qk_norm for gfx950: layer normalisation of every head's 64 query values
// and 64 key values (the DilatedAttention module's qk_norm option: LongNet
// package README, DilatedAttention parameters), with a gain and a bias
// shared by all heads:
//   y = (x - mean) * rstd * gain + bias,  rstd = 1 / sqrt(var + eps),
// mean and the biased variance taken over the row's 64 values. Backward,
// with g = dy * gain and xh = (x - mean) * rstd:
//   dx = rstd * (g - mean(g) - xh * mean(g * xh)),
//   dgain = sum over rows of dy * xh,  dbias = sum over rows of dy.
//
// Rows are HBM-bound work: 8 lanes per row, each moving one 16-byte chunk
// (8 bf16 values; two chunks for fp32), row statistics reduced over the 8
// lanes with xor shuffles. Both tensors go in one launch (the first half of
// the blocks takes q, the second k). The backward recomputes the row
// statistics from x instead of storing them. The gain and bias gradients
// are reduced without atomics: each lane accumulates its 8 columns over the
// rows it visits, each block reduces its lanes in LDS into one partial row
// of 128 floats, and a second kernel adds the partials in a fixed order.
#include <cstring>
#include <type_traits>

#include "da_device.hpp"
#include "kernels.hpp"

namespace da {
namespace {

constexpr int kThreads = 256;
constexpr int kLanesPerRow = 8;
constexpr int kRowsPerPass = kThreads / kLanesPerRow;  // 32
constexpr int kVals = kDh / kLanesPerRow;               // 8 values per lane

template <bool BF>
__device__ inline void load8(const void* base, int64_t elem, float* x) {
  if constexpr (BF) {
    const u32x4 u = *reinterpret_cast<const u32x4*>(reinterpret_cast<const __bf16*>(base) + elem);
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      x[2 * i] = __uint_as_float(u[i] << 16);
      x[2 * i + 1] = __uint_as_float(u[i] & 0xffff0000u);
    }
  } else {
    const f32x4* p = reinterpret_cast<const f32x4*>(reinterpret_cast<const float*>(base) + elem);
    const f32x4 a = p[0], b = p[1];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      x[i] = a[i];
      x[4 + i] = b[i];
    }
  }
}

template <bool BF>
__device__ inline void store8(void* base, int64_t elem, const float* x) {
  if constexpr (BF) {
    *reinterpret_cast<u32x4*>(reinterpret_cast<__bf16*>(base) + elem) =
        u32x4{dev_pack_bf16(x[0], x[1]), dev_pack_bf16(x[2], x[3]), dev_pack_bf16(x[4], x[5]),
              dev_pack_bf16(x[6], x[7])};
  } else {
    f32x4* p = reinterpret_cast<f32x4*>(reinterpret_cast<float*>(base) + elem);
    p[0] = f32x4{x[0], x[1], x[2], x[3]};
    p[1] = f32x4{x[4], x[5], x[6], x[7]};
  }
}

// Sum over the 8 lanes of a row (lanes 8j .. 8j+7 of the wave).
__device__ inline float row_sum(float s) {
  s += __shfl_xor(s, 1);
  s += __shfl_xor(s, 2);
  s += __shfl_xor(s, 4);
  return s;
}

// Row statistics from the lane's 8 values: mean and rstd.
__device__ inline void row_stats(const float* x, float eps, float* mean, float* rstd) {
  float s = 0.f;
#pragma unroll
  for (int i = 0; i < kVals; ++i) s += x[i];
  const float mu = row_sum(s) * (1.f / kDh);
  float v = 0.f;
#pragma unroll
  for (int i = 0; i < kVals; ++i) {
    const float d = x[i] - mu;
    v = fmaf(d, d, v);
  }
  *mean = mu;
  *rstd = __builtin_amdgcn_rsqf(row_sum(v) * (1.f / kDh) + eps);
}

template <bool BF>
__global__ __launch_bounds__(kThreads) void qk_norm_fwd_kernel(const QkNormArgs a) {
  const int which = blockIdx.x >= gridDim.x / 2;  // 0: q, 1: k
  const int64_t blk = blockIdx.x - which * (gridDim.x / 2);
  const int64_t nblk = gridDim.x / 2;
  const void* x = which ? a.xk : a.xq;
  void* y = which ? a.yk : a.yq;
  const int sub = threadIdx.x % kLanesPerRow;
  float gain[kVals], bias[kVals];
  load8<BF>(which ? a.gk : a.gq, kVals * sub, gain);
  load8<BF>(which ? a.bk : a.bq, kVals * sub, bias);
  // every lane of a wave runs the same number of passes (rows of a pass are
  // consecutive), so the shuffles see all 8 lanes of each row
  for (int64_t r0 = blk * kRowsPerPass; r0 < a.rows; r0 += nblk * kRowsPerPass) {
    const int64_t row = r0 + threadIdx.x / kLanesPerRow;
    const bool valid = row < a.rows;
    const int64_t elem = (valid ? row : 0) * kDh + kVals * sub;
    float v[kVals];
    load8<BF>(x, elem, v);
    float mean, rstd;
    row_stats(v, a.eps, &mean, &rstd);
#pragma unroll
    for (int i = 0; i < kVals; ++i) v[i] = fmaf((v[i] - mean) * rstd, gain[i], bias[i]);
    if (valid) store8<BF>(y, elem, v);
  }
}

template <bool BF>
__global__ __launch_bounds__(kThreads) void qk_norm_bwd_kernel(const QkNormArgs a) {
  __shared__ float red[kRowsPerPass][2 * kDh + 1];
  const int which = blockIdx.x >= gridDim.x / 2;
  const int64_t blk = blockIdx.x - which * (gridDim.x / 2);
  const int64_t nblk = gridDim.x / 2;
  const void* x = which ? a.xk : a.xq;
  const void* dy = which ? a.dyk : a.dyq;
  void* dx = which ? a.dxk : a.dxq;
  const int sub = threadIdx.x % kLanesPerRow;
  float gain[kVals];
  load8<BF>(which ? a.gk : a.gq, kVals * sub, gain);
  float acc_g[kVals], acc_b[kVals];
#pragma unroll
  for (int i = 0; i < kVals; ++i) acc_g[i] = acc_b[i] = 0.f;
  // two passes per iteration: both passes' loads are issued before either
  // is used, so their memory latencies overlap
  for (int64_t r0 = blk * kRowsPerPass; r0 < a.rows; r0 += 2 * nblk * kRowsPerPass) {
    float v[2][kVals], d[2][kVals];
    int64_t elem[2];
    bool valid[2];
#pragma unroll
    for (int u = 0; u < 2; ++u) {
      const int64_t row = r0 + u * nblk * kRowsPerPass + threadIdx.x / kLanesPerRow;
      valid[u] = row < a.rows;
      elem[u] = (valid[u] ? row : 0) * kDh + kVals * sub;
      load8<BF>(x, elem[u], v[u]);
      load8<BF>(dy, elem[u], d[u]);
    }
#pragma unroll
    for (int u = 0; u < 2; ++u) {
      if (!valid[u]) {
#pragma unroll
        for (int i = 0; i < kVals; ++i) d[u][i] = 0.f;
      }
      float mean, rstd;
      row_stats(v[u], a.eps, &mean, &rstd);
      float sg = 0.f, sgx = 0.f;
#pragma unroll
      for (int i = 0; i < kVals; ++i) {
        v[u][i] = (v[u][i] - mean) * rstd;  // xh
        const float g = d[u][i] * gain[i];
        sg += g;
        sgx = fmaf(g, v[u][i], sgx);
        acc_g[i] = fmaf(d[u][i], v[u][i], acc_g[i]);
        acc_b[i] += d[u][i];
      }
      const float mg = row_sum(sg) * (1.f / kDh);
      const float mgx = row_sum(sgx) * (1.f / kDh);
      float o[kVals];
#pragma unroll
      for (int i = 0; i < kVals; ++i) o[i] = rstd * (d[u][i] * gain[i] - mg - v[u][i] * mgx);
      if (valid[u]) store8<BF>(dx, elem[u], o);
    }
  }
  // block partial of dgain, dbias: rows of the block's 32 row slots, then
  // the 32 slots in order
  const int slot = threadIdx.x / kLanesPerRow;
#pragma unroll
  for (int i = 0; i < kVals; ++i) {
    red[slot][kVals * sub + i] = acc_g[i];
    red[slot][kDh + kVals * sub + i] = acc_b[i];
  }
  __syncthreads();
  if (threadIdx.x < 2 * kDh) {
    float s = 0.f;
    for (int j = 0; j < kRowsPerPass; ++j) s += red[j][threadIdx.x];
    a.partials[(which * nblk + blk) * (2 * kDh) + threadIdx.x] = s;
  }
}

// dparams[which][0 = gain, 1 = bias][64] = sum over blocks of the partials:
// one block per output element (blockIdx.x = which * 128 + column); thread
// t adds the partials t, t + 256, ... in order, then the block adds the 256
// thread sums in a fixed tree.
__global__ __launch_bounds__(kThreads) void qk_norm_reduce_kernel(const QkNormArgs a, int64_t nblk) {
  __shared__ float part[kThreads];
  const int which = blockIdx.x / (2 * kDh);
  const int col = blockIdx.x % (2 * kDh);
  float s = 0.f;
  for (int64_t b = threadIdx.x; b < nblk; b += kThreads)
    s += a.partials[(which * nblk + b) * (2 * kDh) + col];
  part[threadIdx.x] = s;
  __syncthreads();
  for (int w = kThreads / 2; w > 0; w /= 2) {
    if (threadIdx.x < w) part[threadIdx.x] += part[threadIdx.x + w];
    __syncthreads();
  }
  if (threadIdx.x == 0) a.dparams[blockIdx.x] = part[0];
}

}  // namespace

int64_t qk_norm_blocks(int64_t rows) {
  // blocks per tensor: enough to fill the chip, never more than the passes
  const int64_t passes = (rows + kRowsPerPass - 1) / kRowsPerPass;
  return passes < 1024 ? (passes > 0 ? passes : 1) : 1024;
}

hipError_t launch_qk_norm_fwd(const QkNormArgs& a, bool bf16, hipStream_t st) {
  const dim3 g((uint32_t)(2 * qk_norm_blocks(a.rows))), b(kThreads);
  if (bf16)
    hipLaunchKernelGGL(qk_norm_fwd_kernel<true>, g, b, 0, st, a);
  else
    hipLaunchKernelGGL(qk_norm_fwd_kernel<false>, g, b, 0, st, a);
  return hipGetLastError();
}

hipError_t launch_qk_norm_bwd(const QkNormArgs& a, bool bf16, hipStream_t st) {
  const int64_t nb = qk_norm_blocks(a.rows);
  const dim3 g((uint32_t)(2 * nb)), b(kThreads);
  if (bf16)
    hipLaunchKernelGGL(qk_norm_bwd_kernel<true>, g, b, 0, st, a);
  else
    hipLaunchKernelGGL(qk_norm_bwd_kernel<false>, g, b, 0, st, a);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(qk_norm_reduce_kernel, dim3(2 * 2 * kDh), dim3(kThreads), 0, st, a, nb);
  return hipGetLastError();
}

hipError_t launch_qk_norm_reduce(const float* partials, int64_t nblk, float* dparams,
                                 hipStream_t st) {
  QkNormArgs a;
  memset(&a, 0, sizeof a);
  a.partials = const_cast<float*>(partials);
  a.dparams = dparams;
  hipLaunchKernelGGL(qk_norm_reduce_kernel, dim3(2 * 2 * kDh), dim3(kThreads), 0, st, a, nblk);
  return hipGetLastError();
}

}  // namespace da
