// Fused dilated-attention kernel for gfx950 (MI355X).
//
// One workgroup computes one query tile of one (batch, head, segment) of one
// pattern: it gathers the segment's dilated rows (every r-th position from
// the head's offset: LongNet blog, "LongNet's attention allocation
// principle"; "LongNet论文精读" page, "Dilated Attention的工作原理" steps 1-2),
// runs softmax attention over them (step 3) with an online softmax, and
// writes the rows back to their positions (step 4) or, when several
// patterns are mixed, to per-pattern partial buffers for the merge kernel.
//
// Work decomposition (NW waves of 64 lanes per workgroup):
//   * each wave owns 32 query rows (BM = 32 * NW per workgroup);
//   * key/value tiles of BN gathered rows are staged through LDS, double
//     buffered, loaded by the whole workgroup: K row-major with a 16-byte
//     XOR swizzle, V transposed (d-major) so PV operands are contiguous;
//   * S^T = K Q^T and O^T += V^T P^T run on MFMA 32x32 blocks. With S^T, a
//     lane holds one query and 16 keys of a block, so row max and row sum
//     are in-lane except for one exchange with the lane 32 apart.
// bf16 inputs use v_mfma_f32_32x32x16_bf16 (P rounded to bf16 for PV, the
// row sum taken over the same rounded values); fp32 inputs use
// v_mfma_f32_32x32x2_f32 with P kept in fp32.
#include <type_traits>

#include "da_common.hpp"
#include "kernels.hpp"

namespace da {
namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

constexpr float kLn2 = 0.69314718055994530942f;

struct Tile {
  int64_t b;
  int64_t seg;
  int32_t h;
  int32_t p;    // index into AttnArgs::pat (sorted order)
  int32_t qt;   // query tile inside the segment
};

// Block id -> tile (see AttnArgs for the order). Returns false for the
// padding blocks of XCDs whose list is shorter than the longest one.
__device__ inline bool decode_tile(const AttnArgs& a, int64_t id, Tile* t) {
  const int32_t x = (int32_t)(id % kXcds);
  int64_t slot = id / kXcds;
  for (int p = 0; p < a.np; ++p) {
    const int64_t u0 = a.unit_start[p], u1 = a.unit_start[p + 1];
    // first unit of this pattern dealt to XCD x, and how many it gets
    const int64_t first = u0 + (((x - u0) % kXcds) + kXcds) % kXcds;
    const int64_t cnt = first < u1 ? (u1 - first + kXcds - 1) / kXcds : 0;
    const int64_t nt = a.pat[p].ntile;
    if (slot < cnt * nt) {
      const int64_t lu = slot / nt;
      const int64_t rem = first + lu * kXcds - u0;  // unit index inside the pattern
      const int64_t nseg = a.pat[p].nseg;
      t->seg = rem % nseg;
      const int64_t bh = rem / nseg;
      t->h = (int32_t)(bh % a.H);
      t->b = bh / a.H;
      t->p = p;
      t->qt = (int32_t)(nt - 1 - (slot - lu * nt));
      return true;
    }
    slot -= cnt * nt;
  }
  return false;
}

__device__ inline float exp2_fast(float x) { return __builtin_amdgcn_exp2f(x); }

// Combine a per-lane value with the lane 32 apart (both halves of a query).
__device__ inline float pair_max(float x) {
  auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}
__device__ inline float pair_sum(float x) {
  auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}

template <bool BF, int NW, int BN>
struct Smem {
  // bf16: K [BN][64] swizzled, V^T [64][BN + 4]; fp32: K [BN][65], V [BN][64]
  static constexpr int kVtStride = BN + 4;
  static constexpr int kKElems = BF ? BN * kDh : BN * (kDh + 1);
  static constexpr int kVElems = BF ? kDh * kVtStride : BN * kDh;
  static constexpr int kElemBytes = BF ? 2 : 4;
  static constexpr int kBytes = 2 * (kKElems + kVElems) * kElemBytes;
};

template <int NW, int BN, bool CAUSAL, bool FINAL, bool BF>
__global__ __launch_bounds__(NW * 64) void attn_fwd_kernel(const AttnArgs a) {
  using T = typename std::conditional<BF, __bf16, float>::type;
  using SM = Smem<BF, NW, BN>;
  constexpr int BM = 32 * NW;
  constexpr int NT = 64 * NW;
  constexpr int KB = BN / 32;
  static_assert(BN % 32 == 0 && BN <= 128, "key tile");

  __shared__ __attribute__((aligned(16))) char smem[SM::kBytes];
  T* const Ks = reinterpret_cast<T*>(smem);
  T* const Vs = Ks + 2 * SM::kKElems;

  Tile tl;
  if (!decode_tile(a, blockIdx.x, &tl)) return;
  const PatDev& P = a.pat[tl.p];
  const int32_t r = P.r;
  const int64_t wp = P.wp;
  const int32_t off = head_offset(tl.h, r);
  const int32_t L = rows_gathered(wp, off, r);
  const int32_t q0 = tl.qt * BM;
  if (q0 >= L) return;  // last tile of a head one row shorter than lmax

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wv = tid >> 6;
  const int n = lane & 31;
  const int hh = lane >> 5;

  const int64_t rs = (int64_t)a.H * kDh;  // elements between consecutive positions
  const int64_t seg0 = tl.seg * wp;
  const int64_t headbase = tl.b * a.N * rs + (int64_t)tl.h * kDh;
  // gathered row m starts at element rowbase + m * mstride
  const int64_t rowbase = headbase + gathered_pos(tl.seg, wp, off, r, 0) * rs;
  const int64_t mstride = (int64_t)r * rs;

  const int32_t qend_wg = min(L, q0 + BM);
  const int32_t nkt = CAUSAL ? (qend_wg + BN - 1) / BN : (L + BN - 1) / BN;
  const int32_t qw0 = q0 + wv * 32;
  const int32_t qend_w = min(L, qw0 + 32);
  const int32_t nkt_w = qw0 >= L ? 0 : (CAUSAL ? (qend_w + BN - 1) / BN : nkt);
  const int32_t mq = qw0 + n;  // this lane's query (gathered index)
  const bool qvalid = mq < L;
  // Rows past L are read from row L-1 instead of being skipped: keys past L
  // are masked and queries past L are never stored, so no load needs a branch.
  const int32_t mqc = min(mq, L - 1);

  const T* const Qg = reinterpret_cast<const T*>(a.q);
  const T* const Kg = reinterpret_cast<const T*>(a.k);
  const T* const Vg = reinterpret_cast<const T*>(a.v);

  // ---- query fragments (B operand of S^T = K Q^T), kept in registers
  constexpr int QREGS = BF ? 4 : 32;
  typename std::conditional<BF, bf16x8, float>::type qf[QREGS];
  if constexpr (BF) {
    const T* qrow = Qg + rowbase + (int64_t)mqc * mstride + 8 * hh;
#pragma unroll
    for (int ks = 0; ks < 4; ++ks)
      qf[ks] = __builtin_bit_cast(bf16x8, *reinterpret_cast<const u32x4*>(qrow + 16 * ks));
  } else {
    const T* qrow = Qg + rowbase + (int64_t)mqc * mstride;
#pragma unroll
    for (int c = 0; c < 16; ++c) {
      const f32x4 x = *reinterpret_cast<const f32x4*>(qrow + 4 * c);
      qf[2 * c] = hh ? x[1] : x[0];
      qf[2 * c + 1] = hh ? x[3] : x[2];
    }
  }

  // ---- key/value tile staging: global -> registers -> LDS
  constexpr int CK = BF ? BN * 8 / NT : BN * 16 / NT;  // 16-byte K chunks per thread
  constexpr int CV = BF ? BN * 4 / NT : BN * 16 / NT;  // V items per thread
  static_assert(CK >= 1 && CV >= 1, "tile too small for the workgroup");
  u32x4 kreg[CK];
  u32x2 vreg[BF ? CV : 1][4];
  f32x4 vreg32[BF ? 1 : CV];

  auto load_tile = [&](int kt) {
    const int32_t mbase = kt * BN;
#pragma unroll
    for (int i = 0; i < CK; ++i) {
      const int c = tid + i * NT;
      const int row = BF ? (c >> 3) : (c >> 4);
      const int ch = BF ? (c & 7) : (c & 15);
      const int32_t m = min(mbase + row, L - 1);
      kreg[i] = *reinterpret_cast<const u32x4*>(Kg + rowbase + (int64_t)m * mstride +
                                                 ch * (BF ? 8 : 4));
    }
    if constexpr (BF) {
#pragma unroll
      for (int i = 0; i < CV; ++i) {
        const int c = tid + i * NT;
        const int kg = c >> 4, dg = c & 15;
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          const int32_t m = min(mbase + 4 * kg + j, L - 1);
          vreg[i][j] =
              *reinterpret_cast<const u32x2*>(Vg + rowbase + (int64_t)m * mstride + 4 * dg);
        }
      }
    } else {
#pragma unroll
      for (int i = 0; i < CV; ++i) {
        const int c = tid + i * NT;
        const int row = c >> 4, ch = c & 15;
        const int32_t m = min(mbase + row, L - 1);
        vreg32[i] = *reinterpret_cast<const f32x4*>(Vg + rowbase + (int64_t)m * mstride + 4 * ch);
      }
    }
  };

  auto store_tile = [&](int buf) {
    T* K = Ks + buf * SM::kKElems;
    T* V = Vs + buf * SM::kVElems;
#pragma unroll
    for (int i = 0; i < CK; ++i) {
      const int c = tid + i * NT;
      if constexpr (BF) {
        const int row = c >> 3, ch = c & 7;
        *reinterpret_cast<u32x4*>(K + row * kDh + ((ch ^ (row & 7)) << 3)) = kreg[i];
      } else {
        const int row = c >> 4, ch = c & 15;
        float* dst = reinterpret_cast<float*>(K) + row * (kDh + 1) + 4 * ch;
#pragma unroll
        for (int e = 0; e < 4; ++e) dst[e] = __uint_as_float(kreg[i][e]);
      }
    }
    if constexpr (BF) {
      // 4 keys x 4 dims -> 4 dims x 4 keys (bf16 pairs regrouped)
#pragma unroll
      for (int i = 0; i < CV; ++i) {
        const int c = tid + i * NT;
        const int kg = c >> 4, dg = c & 15;
        const u32x2* x = vreg[i];
        u32x2 o[4];
        o[0] = u32x2{(x[0][0] & 0xffffu) | (x[1][0] << 16), (x[2][0] & 0xffffu) | (x[3][0] << 16)};
        o[1] = u32x2{(x[0][0] >> 16) | (x[1][0] & 0xffff0000u),
                     (x[2][0] >> 16) | (x[3][0] & 0xffff0000u)};
        o[2] = u32x2{(x[0][1] & 0xffffu) | (x[1][1] << 16), (x[2][1] & 0xffffu) | (x[3][1] << 16)};
        o[3] = u32x2{(x[0][1] >> 16) | (x[1][1] & 0xffff0000u),
                     (x[2][1] >> 16) | (x[3][1] & 0xffff0000u)};
#pragma unroll
        for (int e = 0; e < 4; ++e)
          *reinterpret_cast<u32x2*>(V + (4 * dg + e) * SM::kVtStride + 4 * kg) = o[e];
      }
    } else {
#pragma unroll
      for (int i = 0; i < CV; ++i) {
        const int c = tid + i * NT;
        const int row = c >> 4, ch = c & 15;
        *reinterpret_cast<f32x4*>(reinterpret_cast<float*>(V) + row * kDh + 4 * ch) = vreg32[i];
      }
    }
  };

  // ---- running state: O^T accumulators (2 blocks of 32 dims), row max
  // (log2 domain, identical in both lane halves) and this half's row sum
  f32x16 O[2];
#pragma unroll
  for (int db = 0; db < 2; ++db)
#pragma unroll
    for (int v = 0; v < 16; ++v) O[db][v] = 0.f;
  float m_run = -INFINITY;
  float l_run = 0.f;
  const float sl2 = a.sl2;

  auto compute = [&](int buf, int kt) {
    const T* K = Ks + buf * SM::kKElems;
    const T* V = Vs + buf * SM::kVElems;
    f32x16 S[KB];
#pragma unroll
    for (int kb = 0; kb < KB; ++kb) {
#pragma unroll
      for (int v = 0; v < 16; ++v) S[kb][v] = 0.f;
      const int row = kb * 32 + n;
      if constexpr (BF) {
#pragma unroll
        for (int ks = 0; ks < 4; ++ks) {
          const bf16x8 kf = *reinterpret_cast<const bf16x8*>(
              K + row * kDh + (((2 * ks + hh) ^ (n & 7)) << 3));
          S[kb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(kf, qf[ks], S[kb], 0, 0, 0);
        }
      } else {
        const float* Kr = reinterpret_cast<const float*>(K) + row * (kDh + 1) + hh;
#pragma unroll
        for (int ks = 0; ks < 32; ++ks)
          S[kb] = __builtin_amdgcn_mfma_f32_32x32x2f32(Kr[2 * ks], qf[ks], S[kb], 0, 0, 0);
      }
    }

    // mask: keys after the query (causal) or past the segment's rows
    const bool need_mask = CAUSAL ? (kt * BN + BN - 1 > qw0) : ((kt + 1) * BN > L);
    if (need_mask) {
#pragma unroll
      for (int kb = 0; kb < KB; ++kb)
#pragma unroll
        for (int v = 0; v < 16; ++v) {
          const int32_t key = kt * BN + kb * 32 + 8 * (v >> 2) + 4 * hh + (v & 3);
          const bool dead = CAUSAL ? (key > mq) : (key >= L);
          if (dead) S[kb][v] = -INFINITY;
        }
    }

    float mx = -INFINITY;
#pragma unroll
    for (int kb = 0; kb < KB; ++kb)
#pragma unroll
      for (int v = 0; v < 16; ++v) mx = fmaxf(mx, S[kb][v]);
    mx = pair_max(mx);
    // Lazy rescaling: the running max (log2 domain) only moves when some row
    // of the wave gains more than 8, so p = 2^(s - m_run) stays below 2^8
    // and most tiles skip rescaling O and l.
    const float mt = mx * sl2;
    if (__ballot(mt > m_run + 8.f) != 0) {
      const float m_new = fmaxf(m_run, mt);
      const float alpha = exp2_fast(m_run - m_new);
      m_run = m_new;
      l_run *= alpha;
#pragma unroll
      for (int db = 0; db < 2; ++db) O[db] *= alpha;
    }

    float lsum = 0.f;
    if constexpr (BF) {
      bf16x8 pb[2 * KB];
#pragma unroll
      for (int c = 0; c < 2 * KB; ++c) {
#pragma unroll
        for (int e = 0; e < 8; e += 2) {
          const float p0 = exp2_fast(fmaf(S[c >> 1][8 * (c & 1) + e], sl2, -m_run));
          const float p1 = exp2_fast(fmaf(S[c >> 1][8 * (c & 1) + e + 1], sl2, -m_run));
          bf16x2 pr;
          pr[0] = (__bf16)p0;
          pr[1] = (__bf16)p1;
          pb[c][e] = pr[0];
          pb[c][e + 1] = pr[1];
          const bf16x2 one2 = {(__bf16)1.0f, (__bf16)1.0f};
          lsum = __builtin_amdgcn_fdot2_f32_bf16(pr, one2, lsum, false);
        }
      }
      l_run += lsum;
#pragma unroll
      for (int db = 0; db < 2; ++db) {
        const T* Vr = V + (db * 32 + n) * SM::kVtStride + 4 * hh;
#pragma unroll
        for (int c = 0; c < 2 * KB; ++c) {
          const u32x2 lo = *reinterpret_cast<const u32x2*>(Vr + 16 * c);
          const u32x2 hi = *reinterpret_cast<const u32x2*>(Vr + 16 * c + 8);
          const bf16x8 vf = __builtin_bit_cast(bf16x8, u32x4{lo[0], lo[1], hi[0], hi[1]});
          O[db] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(vf, pb[c], O[db], 0, 0, 0);
        }
      }
    } else {
      float pf[KB][16];
#pragma unroll
      for (int kb = 0; kb < KB; ++kb)
#pragma unroll
        for (int v = 0; v < 16; ++v) {
          pf[kb][v] = exp2_fast(fmaf(S[kb][v], sl2, -m_run));
          lsum += pf[kb][v];
        }
      l_run += lsum;
#pragma unroll
      for (int db = 0; db < 2; ++db)
#pragma unroll
        for (int kb = 0; kb < KB; ++kb)
#pragma unroll
          for (int v = 0; v < 16; ++v) {
            const int key = kb * 32 + 8 * (v >> 2) + 4 * hh + (v & 3);
            const float vv = reinterpret_cast<const float*>(V)[key * kDh + db * 32 + n];
            O[db] = __builtin_amdgcn_mfma_f32_32x32x2f32(vv, pf[kb][v], O[db], 0, 0, 0);
          }
    }
  };

  // ---- main loop over key tiles, double-buffered through LDS
  load_tile(0);
  store_tile(0);
  __syncthreads();
  for (int kt = 0; kt < nkt; ++kt) {
    const int buf = kt & 1;
    if (kt + 1 < nkt) load_tile(kt + 1);
    if (kt < nkt_w) compute(buf, kt);
    if (kt + 1 < nkt) store_tile(buf ^ 1);
    __syncthreads();
  }

  if (!qvalid) return;
  const float l_tot = pair_sum(l_run);
  const float inv = 1.f / l_tot;
  const float lse2 = m_run + __log2f(l_tot);
  const int64_t pos = gathered_pos(tl.seg, wp, off, r, mq);

  if constexpr (FINAL) {
    T* orow = reinterpret_cast<T*>(a.out) + headbase;
    float* lse_row = a.lse + ((int64_t)tl.b * a.H + tl.h) * a.N;
    auto put = [&](int64_t t, bool zero) {
      T* dst = orow + t * rs + 4 * hh;
#pragma unroll
      for (int db = 0; db < 2; ++db)
#pragma unroll
        for (int g = 0; g < 4; ++g) {
          const int d = db * 32 + 8 * g;
          if constexpr (BF) {
            bf16x2 x0, x1;
            x0[0] = (__bf16)(zero ? 0.f : O[db][4 * g + 0] * inv);
            x0[1] = (__bf16)(zero ? 0.f : O[db][4 * g + 1] * inv);
            x1[0] = (__bf16)(zero ? 0.f : O[db][4 * g + 2] * inv);
            x1[1] = (__bf16)(zero ? 0.f : O[db][4 * g + 3] * inv);
            *reinterpret_cast<u32x2*>(dst + d) =
                u32x2{__builtin_bit_cast(uint32_t, x0), __builtin_bit_cast(uint32_t, x1)};
          } else {
            f32x4 x;
#pragma unroll
            for (int e = 0; e < 4; ++e) x[e] = zero ? 0.f : O[db][4 * g + e] * inv;
            *reinterpret_cast<f32x4*>(dst + d) = x;
          }
        }
      if (hh == 0) lse_row[t] = zero ? -INFINITY : lse2 * kLn2;
    };
    put(pos, false);
    // positions of this segment that the head does not gather: the r-1
    // after each gathered row and, before the first one, the offset rows
    const int64_t seg_end = seg0 + wp;
    for (int j = 1; j < r; ++j) {
      if (pos + j >= seg_end) break;
      put(pos + j, true);
    }
    if (mq == 0)
      for (int j = 0; j < off; ++j) put(seg0 + j, true);
  } else {
    const int64_t prow = (((int64_t)tl.b * a.H + tl.h) * P.nseg + tl.seg) * P.lmax + mq;
    float* po = a.ws + P.po_off + prow * kDh + 4 * hh;
#pragma unroll
    for (int db = 0; db < 2; ++db)
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        f32x4 x;
#pragma unroll
        for (int e = 0; e < 4; ++e) x[e] = O[db][4 * g + e] * inv;
        *reinterpret_cast<f32x4*>(po + db * 32 + 8 * g) = x;
      }
    if (hh == 0) a.ws[P.pl_off + prow] = lse2;
  }
}

template <int NW, int BN, bool BF>
hipError_t launch_nw(const AttnArgs& a, bool causal, bool final_out, int64_t grid,
                     hipStream_t st) {
  dim3 g((uint32_t)grid), b(NW * 64);
  if (causal) {
    if (final_out)
      hipLaunchKernelGGL((attn_fwd_kernel<NW, BN, true, true, BF>), g, b, 0, st, a);
    else
      hipLaunchKernelGGL((attn_fwd_kernel<NW, BN, true, false, BF>), g, b, 0, st, a);
  } else {
    if (final_out)
      hipLaunchKernelGGL((attn_fwd_kernel<NW, BN, false, true, BF>), g, b, 0, st, a);
    else
      hipLaunchKernelGGL((attn_fwd_kernel<NW, BN, false, false, BF>), g, b, 0, st, a);
  }
  return hipGetLastError();
}

}  // namespace

int attn_tile_rows(int nw) { return 32 * nw; }

hipError_t launch_attention(const AttnArgs& a, bool bf16, int nw, bool causal, bool final_out,
                            int64_t grid, hipStream_t st) {
  if (bf16) {
    if (nw == 4) return launch_nw<4, 64, true>(a, causal, final_out, grid, st);
    return launch_nw<1, 32, true>(a, causal, final_out, grid, st);
  }
  if (nw == 4) return launch_nw<4, 64, false>(a, causal, final_out, grid, st);
  return launch_nw<1, 32, false>(a, causal, final_out, grid, st);
}

}  // namespace da
