// Pattern merge for gfx950: combines the per-pattern partial outputs of
// every row with weights exp(lse_i - LSE), LSE = log sum_i exp(lse_i), over
// the patterns that gather the row. The pages describe the mixture of
// patterns ("a series of attention patterns": LongNet blog, "LongNet's
// attention allocation principle"; dakule.com page, "如何做到？") but not
// its weights; weighting by each pattern's softmax denominator is the
// reading implemented here. Rows no pattern gathers get 0 and -inf.
//
// The partials hold log2-domain lse values. Rows gathered by exactly one
// pattern are final after the attention kernel and are skipped here. The
// kernel is bound by HBM traffic: 4 lanes cooperate on one 64-wide row, each
// moving 64 contiguous bytes of every covering pattern's partial, so one
// wave handles 16 rows and the per-row coverage tests are shared by 4 lanes.
// Every covering pattern's lse and partial row are loaded before any is
// used (one memory round trip per row, not one per pattern); the kernel is
// instantiated per pattern count so the registers fit the loads.
#include "da_common.hpp"
#include "kernels.hpp"

namespace da {
namespace {

typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));

constexpr float kLn2 = 0.69314718055994530942f;
constexpr int kLanesPerRow = 4;
constexpr int kDimsPerLane = kDh / kLanesPerRow;  // 16
constexpr int kThreads = 256;
constexpr int kRowsPerBlock = kThreads / kLanesPerRow;  // 64

__device__ inline uint32_t pack_bf16(float x, float y) {
  bf16x2 p;
  p[0] = (__bf16)x;
  p[1] = (__bf16)y;
  return __builtin_bit_cast(uint32_t, p);
}

template <bool BF, int NP>
__global__ __launch_bounds__(kThreads) void merge_kernel(const MergeArgs a, const FastDiv n_div) {
  // blockIdx.y = batch; rows of one batch are taken head by head (h, t), so
  // a block's rows are consecutive positions of one head: each pattern's
  // partial rows and the lse values are then contiguous runs
  const uint32_t row = blockIdx.x * kRowsPerBlock + (threadIdx.x / kLanesPerRow);
  const int sub = threadIdx.x % kLanesPerRow;
  if (row >= (uint32_t)(a.N * a.H)) return;
  const int32_t h = (int32_t)fdiv(row, n_div);
  const uint32_t t = row - (uint32_t)h * (uint32_t)a.N;
  const int64_t b = blockIdx.y;

  // rows exactly one pattern gathers were written by the attention kernel
  int32_t ci[NP];
  int cover = 0;
#pragma unroll
  for (int i = 0; i < NP; ++i) {
    ci[i] = (int32_t)compact_index(t, a.pat[i], head_offset(h, a.pat[i].r));
    cover += ci[i] >= 0;
  }
  if (cover == 1) return;

  // every covering pattern's lse and partial row are loaded before any of
  // them is used, so their memory latencies overlap
  float l[NP];
  f32x4 src[NP][4];
#pragma unroll
  for (int i = 0; i < NP; ++i) {
    l[i] = -INFINITY;
    if (ci[i] >= 0) {
      const PatDev& P = a.pat[i];
      // rows of one batch hold fewer than 2^31 slots (N * H < 2^31)
      const int64_t prow = (b * a.H + h) * P.nseg * P.lmax + ci[i];
      l[i] = a.ws[P.pl_off + prow];
      const f32x4* p =
          reinterpret_cast<const f32x4*>(a.ws + P.po_off + prow * kDh + kDimsPerLane * sub);
#pragma unroll
      for (int j = 0; j < 4; ++j) src[i][j] = p[j];
    }
  }
  float mx = -INFINITY;
#pragma unroll
  for (int i = 0; i < NP; ++i) mx = fmaxf(mx, l[i]);
  f32x4 acc[4] = {};
  float lse = -INFINITY;
  if (mx != -INFINITY) {
    float s = 0.f;
#pragma unroll
    for (int i = 0; i < NP; ++i)
      if (ci[i] >= 0) s += __builtin_amdgcn_exp2f(l[i] - mx);
    const float lse2 = mx + __builtin_amdgcn_logf(s);
#pragma unroll
    for (int i = 0; i < NP; ++i) {
      if (ci[i] < 0) continue;
      const float wgt = __builtin_amdgcn_exp2f(l[i] - lse2);
#pragma unroll
      for (int j = 0; j < 4; ++j) acc[j] += wgt * src[i][j];
    }
    lse = lse2 * kLn2;
  }
  const int64_t orow = (b * a.N + t) * a.H + h;
  if constexpr (BF) {
    u32x4* dst = reinterpret_cast<u32x4*>(reinterpret_cast<__bf16*>(a.out) + orow * kDh +
                                          kDimsPerLane * sub);
#pragma unroll
    for (int j = 0; j < 2; ++j)
      dst[j] = u32x4{pack_bf16(acc[2 * j][0], acc[2 * j][1]), pack_bf16(acc[2 * j][2], acc[2 * j][3]),
                     pack_bf16(acc[2 * j + 1][0], acc[2 * j + 1][1]),
                     pack_bf16(acc[2 * j + 1][2], acc[2 * j + 1][3])};
  } else {
    f32x4* dst = reinterpret_cast<f32x4*>(reinterpret_cast<float*>(a.out) + orow * kDh +
                                          kDimsPerLane * sub);
#pragma unroll
    for (int j = 0; j < 4; ++j) dst[j] = acc[j];
  }
  if (sub == 0) a.lse[(b * a.H + h) * a.N + t] = lse;
}

__global__ void gather_map_kernel(const PatDev p, int32_t h, int64_t* out) {
  const int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (i >= p.nseg * p.lmax) return;
  const int64_t s = i / p.lmax;
  const int32_t m = (int32_t)(i - s * p.lmax);
  const int32_t off = head_offset(h, p.r);
  out[i] = m < rows_gathered(p.wp, off, p.r) ? gathered_pos(s, p.wp, off, p.r, m) : -1;
}

__global__ void coverage_map_kernel(const PatDev p, int32_t h, int64_t N, int64_t* out) {
  const int64_t t = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (t >= N) return;
  out[t] = compact_index((uint32_t)t, p, head_offset(h, p.r));
}

template <bool BF, int NP = 1>
hipError_t launch_merge_np(const MergeArgs& a, dim3 g, dim3 b, const FastDiv& hd, hipStream_t st) {
  if constexpr (NP < kMaxPat) {
    if (a.np > NP) return launch_merge_np<BF, NP + 1>(a, g, b, hd, st);
  }
  hipLaunchKernelGGL((merge_kernel<BF, NP>), g, b, 0, st, a, hd);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_merge(const MergeArgs& a, bool bf16, hipStream_t st) {
  const int64_t rows = a.N * a.H;
  dim3 g((uint32_t)((rows + kRowsPerBlock - 1) / kRowsPerBlock), (uint32_t)a.B), b(kThreads);
  const FastDiv hd = make_fastdiv((uint32_t)a.N);
  return bf16 ? launch_merge_np<true>(a, g, b, hd, st) : launch_merge_np<false>(a, g, b, hd, st);
}

hipError_t launch_gather_map(const PatDev& p, int32_t h, int64_t* out, hipStream_t st) {
  const int64_t n = p.nseg * p.lmax;
  hipLaunchKernelGGL(gather_map_kernel, dim3((uint32_t)((n + 255) / 256)), dim3(256), 0, st, p, h,
                     out);
  return hipGetLastError();
}

hipError_t launch_coverage_map(const PatDev& p, int32_t h, int64_t N, int64_t* out,
                               hipStream_t st) {
  hipLaunchKernelGGL(coverage_map_kernel, dim3((uint32_t)((N + 255) / 256)), dim3(256), 0, st, p,
                     h, N, out);
  return hipGetLastError();
}

}  // namespace da
