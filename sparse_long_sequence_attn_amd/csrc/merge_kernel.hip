// Pattern merge for gfx950: combines the per-pattern partial outputs of
// every row with weights exp(lse_i - LSE), LSE = log sum_i exp(lse_i), over
// the patterns that gather the row. The pages describe the mixture of
// patterns ("a series of attention patterns": LongNet blog, "LongNet's
// attention allocation principle"; dakule.com page, "如何做到？") but not
// its weights; weighting by each pattern's softmax denominator is the
// reading implemented here. Rows no pattern gathers get 0 and -inf.
//
// The partials hold log2-domain lse values. The kernel is bound by HBM
// traffic: 16 lanes cooperate on one 64-wide row with 16-byte loads.
#include "da_common.hpp"
#include "kernels.hpp"

namespace da {
namespace {

typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));

constexpr float kLn2 = 0.69314718055994530942f;
constexpr int kRowsPerBlock = 16;

template <bool BF>
__global__ __launch_bounds__(256) void merge_kernel(const MergeArgs a, const FastDiv h_div) {
  // blockIdx.y = batch; rows of one batch are (t, h) pairs in output order
  const uint32_t row = blockIdx.x * kRowsPerBlock + (threadIdx.x >> 4);
  const int sub = threadIdx.x & 15;
  if (row >= (uint32_t)(a.N * a.H)) return;
  const uint32_t t = fdiv(row, h_div);
  const int32_t h = (int32_t)(row - t * (uint32_t)a.H);
  const int64_t b = blockIdx.y;

  float l[kMaxPat];
  f32x4 o[kMaxPat];
  float mx = -INFINITY;
#pragma unroll
  for (int i = 0; i < kMaxPat; ++i) {
    l[i] = -INFINITY;
    o[i] = f32x4{0.f, 0.f, 0.f, 0.f};
    if (i < a.np) {
      const PatDev& P = a.pat[i];
      const int64_t ci = compact_index(t, P, head_offset(h, P.r));
      if (ci >= 0) {
        const int64_t prow = (b * a.H + h) * P.nseg * P.lmax + ci;
        l[i] = a.ws[P.pl_off + prow];
        o[i] = *reinterpret_cast<const f32x4*>(a.ws + P.po_off + prow * kDh + 4 * sub);
        mx = fmaxf(mx, l[i]);
      }
    }
  }
  f32x4 acc = {0.f, 0.f, 0.f, 0.f};
  float lse = -INFINITY;
  if (mx != -INFINITY) {
    float s = 0.f;
#pragma unroll
    for (int i = 0; i < kMaxPat; ++i) s += exp2f(l[i] - mx);
    const float lse2 = mx + log2f(s);
#pragma unroll
    for (int i = 0; i < kMaxPat; ++i) acc += exp2f(l[i] - lse2) * o[i];
    lse = lse2 * kLn2;
  }
  const int64_t orow = (b * a.N + t) * a.H + h;
  if constexpr (BF) {
    bf16x2 x0, x1;
    x0[0] = (__bf16)acc[0];
    x0[1] = (__bf16)acc[1];
    x1[0] = (__bf16)acc[2];
    x1[1] = (__bf16)acc[3];
    *reinterpret_cast<u32x2*>(reinterpret_cast<__bf16*>(a.out) + orow * kDh + 4 * sub) =
        u32x2{__builtin_bit_cast(uint32_t, x0), __builtin_bit_cast(uint32_t, x1)};
  } else {
    *reinterpret_cast<f32x4*>(reinterpret_cast<float*>(a.out) + orow * kDh + 4 * sub) = acc;
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

}  // namespace

hipError_t launch_merge(const MergeArgs& a, bool bf16, hipStream_t st) {
  const int64_t rows = a.N * a.H;
  dim3 g((uint32_t)((rows + kRowsPerBlock - 1) / kRowsPerBlock), (uint32_t)a.B), b(256);
  const FastDiv hd = make_fastdiv((uint32_t)a.H);
  if (bf16)
    hipLaunchKernelGGL(merge_kernel<true>, g, b, 0, st, a, hd);
  else
    hipLaunchKernelGGL(merge_kernel<false>, g, b, 0, st, a, hd);
  return hipGetLastError();
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
