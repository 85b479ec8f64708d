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
// used (one memory round trip per row, not one per pattern); the kernels
// are instantiated per pattern count so the registers fit the loads.
//
// When some pattern has dilation 1 every position is gathered, and only
// rows with two or more covering patterns need work: merge_pairs_kernel
// lays its threads over the gathered rows of the patterns that can be a
// row's second cover, so no lane idles on a row the attention kernel has
// already finished (with the usual nested dilations 1, 2, 4, ... half of
// all rows). Otherwise merge_kernel takes every position, including the
// rows no pattern gathers.
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
constexpr int kVecPerLane = kDimsPerLane / 4;      // float4 loads per partial row
constexpr int kThreads = 128;
constexpr int kRowsPerBlock = kThreads / kLanesPerRow;  // 32

__device__ inline uint32_t pack_bf16(float x, float y) {
  bf16x2 p;
  p[0] = (__bf16)x;
  p[1] = (__bf16)y;
  return __builtin_bit_cast(uint32_t, p);
}

// Slot of position t among the gathered rows of pattern P for head h
// (s * lmax + m), or -1: t is gathered row m of segment s when
// rel = (t mod w') - (h mod r) is >= 0 and a multiple of r. Branch-free.
__device__ inline int32_t slot_of(const PatDev& P, uint32_t t, uint32_t h) {
  const uint32_t s = fdiv(t, P.wp_div);
  const uint32_t off = h - fdiv(h, P.r_div) * (uint32_t)P.r;
  const int32_t rel = (int32_t)(t - s * P.wp_div.d) - (int32_t)off;
  const uint32_t m = fdiv((uint32_t)rel, P.r_div);  // only meaningful for rel >= 0
  const bool cov = rel >= 0 && (uint32_t)rel == m * (uint32_t)P.r;
  return cov ? (int32_t)(s * (uint32_t)P.lmax + m) : -1;
}

// Merges position t of head h in batch b from the partials of the patterns
// with ci[i] >= 0 (their slots); this lane moves dims 16 sub .. + 15. Every
// covering pattern's lse and partial row are loaded before any of them is
// used, so their memory latencies overlap.
template <bool BF, int NP>
__device__ inline void merge_row(const MergeArgs& a, int64_t b, uint32_t h, uint32_t t, int sub,
                                 const int32_t (&ci)[NP]) {
  float l[NP];
  f32x4 src[NP][kVecPerLane];
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
      for (int j = 0; j < kVecPerLane; ++j) src[i][j] = p[j];
    }
  }
  float mx = -INFINITY;
#pragma unroll
  for (int i = 0; i < NP; ++i) mx = fmaxf(mx, l[i]);
  f32x4 acc[kVecPerLane] = {};
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
      for (int j = 0; j < kVecPerLane; ++j) acc[j] += wgt * src[i][j];
    }
    lse = lse2 * kLn2;
  }
  const int64_t orow = (b * a.N + t) * a.H + h;
  if constexpr (BF) {
    u32x4* dst = reinterpret_cast<u32x4*>(reinterpret_cast<__bf16*>(a.out) + orow * kDh +
                                          kDimsPerLane * sub);
#pragma unroll
    for (int j = 0; j < kVecPerLane / 2; ++j)
      dst[j] = u32x4{pack_bf16(acc[2 * j][0], acc[2 * j][1]), pack_bf16(acc[2 * j][2], acc[2 * j][3]),
                     pack_bf16(acc[2 * j + 1][0], acc[2 * j + 1][1]),
                     pack_bf16(acc[2 * j + 1][2], acc[2 * j + 1][3])};
  } else {
    f32x4* dst = reinterpret_cast<f32x4*>(reinterpret_cast<float*>(a.out) + orow * kDh +
                                          kDimsPerLane * sub);
#pragma unroll
    for (int j = 0; j < kVecPerLane; ++j) dst[j] = acc[j];
  }
  if (sub == 0) a.lse[(b * a.H + h) * a.N + t] = lse;
}

// Every position: 4 lanes per position, positions taken head by head
// (blockIdx.y = batch), so a block's rows are consecutive positions of one
// head and each pattern's partial rows and the lse values are contiguous
// runs. Rows exactly one pattern gathers were written by the attention
// kernel and are skipped; rows no pattern gathers get 0 and -inf.
template <bool BF, int NP>
__global__ __launch_bounds__(kThreads) void merge_kernel(const MergeArgs a, const FastDiv n_div) {
  const uint32_t row = blockIdx.x * kRowsPerBlock + (threadIdx.x / kLanesPerRow);
  const int sub = threadIdx.x % kLanesPerRow;
  if (row >= (uint32_t)(a.N * a.H)) return;
  const uint32_t h = fdiv(row, n_div);
  const uint32_t t = row - h * (uint32_t)a.N;
  int32_t ci[NP];
  int cover = 0;
#pragma unroll
  for (int i = 0; i < NP; ++i) {
    ci[i] = slot_of(a.pat[i], t, h);
    cover += ci[i] >= 0;
  }
  if (cover == 1) return;
  merge_row<BF, NP>(a, blockIdx.y, h, t, sub, ci);
}

// Only rows that need a merge: 4 lanes per gathered row of an enumerated
// pattern j (the partial buffer's slot order, so j's partial rows are read
// as one contiguous run); the row is merged here when j is its second
// covering pattern in rank order, which holds for exactly one enumerating
// thread of every row with two or more covering patterns. Patterns that
// cannot be anyone's second cover are not enumerated (launcher).
template <bool BF, int NP>
__global__ __launch_bounds__(kThreads) void merge_pairs_kernel(const MergeArgs a) {
  const uint32_t blk = blockIdx.x;
  int e = 0;
  while (e + 1 < a.nenum && blk >= a.enum_blk[e + 1]) ++e;
  const int j = a.enum_pat[e];
  const PatDev& P = a.pat[j];
  const uint32_t slot = (blk - a.enum_blk[e]) * kRowsPerBlock + threadIdx.x / kLanesPerRow;
  const int sub = threadIdx.x % kLanesPerRow;
  const uint32_t per_head = a.enum_head_div[e].d;  // nseg * lmax
  if (slot >= (uint32_t)a.H * per_head) return;
  const uint32_t h = fdiv(slot, a.enum_head_div[e]);
  const uint32_t rem = slot - h * per_head;
  const uint32_t s = fdiv(rem, a.enum_lmax_div[e]);
  const uint32_t m = rem - s * (uint32_t)P.lmax;
  const uint32_t off = h - fdiv(h, P.r_div) * (uint32_t)P.r;
  const uint32_t in_seg = off + m * (uint32_t)P.r;
  if (in_seg >= (uint32_t)P.wp) return;  // padding slot of a head with offset > 0
  const uint32_t t = s * (uint32_t)P.wp + in_seg;
  int32_t ci[NP];
  int before = 0;
#pragma unroll
  for (int i = 0; i < NP; ++i) {
    ci[i] = i == j ? (int32_t)rem : slot_of(a.pat[i], t, h);
    before += ci[i] >= 0 && a.rank[i] < a.rank[j];
  }
  if (before != 1) return;
  merge_row<BF, NP>(a, blockIdx.y, h, t, sub, ci);
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
  if (a.nenum > 0)
    hipLaunchKernelGGL((merge_pairs_kernel<BF, NP>), g, b, 0, st, a);
  else
    hipLaunchKernelGGL((merge_kernel<BF, NP>), g, b, 0, st, a, hd);
  return hipGetLastError();
}

// Pattern i gathers, for every head, every position pattern j gathers:
// with r_i | r_j, r_j | w'_j and r_i | w'_i, a row of j at t = s w'_j +
// (h mod r_j) + m r_j has t mod r_i = h mod r_i = (t mod w'_i) mod r_i.
bool covers(const PatDev& i, const PatDev& j) {
  return j.r % i.r == 0 && j.wp % j.r == 0 && i.wp % i.r == 0;
}

}  // namespace

hipError_t launch_merge(const MergeArgs& args, bool bf16, hipStream_t st) {
  MergeArgs a = args;
  // rank by dilation (stable): the densest pattern first
  int order[kMaxPat];
  for (int i = 0; i < a.np; ++i) order[i] = i;
  for (int i = 1; i < a.np; ++i)
    for (int k = i; k > 0 && a.pat[order[k]].r < a.pat[order[k - 1]].r; --k) {
      const int x = order[k];
      order[k] = order[k - 1];
      order[k - 1] = x;
    }
  for (int k = 0; k < a.np; ++k) a.rank[order[k]] = k;
  // a pattern with r = 1 gathers every position, so no row is left for the
  // zero fill and only rows with two or more covering patterns need a thread
  bool all_covered = false;
  for (int i = 0; i < a.np; ++i) all_covered |= a.pat[i].r == 1;
  a.nenum = 0;
  uint32_t blocks = 0;
  if (all_covered) {
    for (int k = 1; k < a.np; ++k) {
      const PatDev& J = a.pat[order[k]];
      int full = 0;  // earlier patterns that gather all of J's rows
      for (int q = 0; q < k; ++q) full += covers(a.pat[order[q]], J);
      if (full >= 2) continue;  // J is never a row's second cover
      const uint32_t per_head = (uint32_t)(J.nseg * J.lmax);
      a.enum_pat[a.nenum] = order[k];
      a.enum_blk[a.nenum] = blocks;
      a.enum_head_div[a.nenum] = make_fastdiv(per_head);
      a.enum_lmax_div[a.nenum] = make_fastdiv((uint32_t)J.lmax);
      ++a.nenum;
      blocks += (uint32_t)(((int64_t)a.H * per_head + kRowsPerBlock - 1) / kRowsPerBlock);
    }
    a.enum_blk[a.nenum] = blocks;
  }
  const int64_t rows = a.N * a.H;
  dim3 g(a.nenum > 0 ? blocks : (uint32_t)((rows + kRowsPerBlock - 1) / kRowsPerBlock),
         (uint32_t)a.B),
      b(kThreads);
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
