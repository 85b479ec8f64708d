// Shared host/device definitions of the dilated-attention library:
// per-launch parameter blocks and the one index function that every kernel
// (attention, merge, map dumps) uses to place gathered rows.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace da {

constexpr int kDh = 64;       // head dimension the kernels are built for
constexpr int kMaxPat = 8;    // patterns per call

// Unsigned 32-bit division by a run-time constant d >= 1 as a multiply-high,
// add and shift (round-up method of Granlund and Montgomery, "Division by
// Invariant Integers using Multiplication", PLDI 1994): with s = ceil(log2 d)
// and m = floor(2^32 (2^s - d) / d) + 1, n / d = (mulhi(n, m) + n) >> s for
// every n < 2^32 when the addition is carried out in 64 bits.
struct FastDiv {
  uint32_t d;
  uint32_t m;
  uint32_t s;
  uint32_t pad_;
};

inline FastDiv make_fastdiv(uint32_t d) {
  uint32_t s = 0;
  while (s < 32 && (uint64_t(1) << s) < d) ++s;
  const uint64_t m = ((uint64_t(1) << 32) * ((uint64_t(1) << s) - d)) / d + 1;
  return FastDiv{d, (uint32_t)m, s, 0};
}

__host__ __device__ inline uint32_t fdiv(uint32_t n, const FastDiv& f) {
  const uint64_t hi = ((uint64_t)n * f.m) >> 32;
  return (uint32_t)((hi + n) >> f.s);
}

// One pattern after planning. Geometry follows the segment / dilation /
// per-head-offset construction of the LongNet blog ("LongNet's attention
// allocation principle" and the multi-head paragraph after it).
struct PatDev {
  int64_t wp;      // effective segment length min(w, N)
  int64_t nseg;    // N / wp
  int64_t units;   // B * H * nseg independent (batch, head, segment) problems
  int64_t po_off;  // float offset of this pattern's partial outputs in the workspace
  int64_t pl_off;  // float offset of this pattern's partial log2-sum-exp values
  int32_t r;       // dilation rate
  int32_t lmax;    // ceil(wp / r): rows gathered by a head with offset 0
  int32_t ntile;   // query tiles per segment: ceil(lmax / BM)
  int32_t group;   // units per group of the tile order (set per launch)
  FastDiv wp_div;  // division by wp
  FastDiv r_div;   // division by r
  // set per launch by the host for the tile order below
  FastDiv nseg_div;  // division by nseg
  FastDiv g_div;     // division by group
  FastDiv grp_div;   // division by group * ntile (one group's tiles)
};

// Attention launch. Tiles of all patterns share one grid. Block ids are
// dealt to the chip's XCDs round-robin (id mod kXcds), so the tiles are laid
// out per XCD: each XCD gets its share of every pattern's (batch, head,
// segment) units and walks them in groups of 4 units, heaviest tiles of the
// group first (the last query tile of each unit, then the one before it,
// and so on); the last pattern's groups are larger (up to what its units'
// key/value rows need of the XCD's 4 MiB L2). A group's key/value rows
// about fill the L2, and the list ends with its shortest tiles, so the
// XCD's workgroup slots drain together instead of waiting on the long
// tiles of the final units. Patterns are
// stored sorted by ntile (descending); units are handed to XCDs round-robin
// in that order.
constexpr int kXcds = 8;

struct AttnArgs {
  FastDiv h_div;   // division by H
  const void* q;
  const void* k;
  const void* v;
  void* out;       // final output (single pattern) - unused otherwise
  float* lse;      // final lse (single pattern) - unused otherwise
  float* ws;       // workspace partials (two or more patterns)
  int64_t B;
  int64_t N;
  int32_t H;
  int32_t np;
  float sl2;       // softmax scale * log2(e)
  float qkn_eps;   // qk_norm fused into the loads (one-wave kernel): epsilon
  // qk_norm fused: gain_q, bias_q, gain_k, bias_k (Dh values each, q's dtype);
  // q and k then hold the un-normalised rows
  const void* qkn[4];
  // qk_norm fused: elements between consecutive positions of q, k and v (at
  // least H * Dh; they may interleave in one buffer); out stays [B, N, H, Dh]
  int64_t in_rs;
  PatDev pat[kMaxPat];
  int64_t unit_start[kMaxPat + 1];  // first global unit of each sorted pattern
};

// Single-launch forward: the patterns' merge folded into one online
// softmax. With reading R1 a row's merged output is one softmax over every
// (pattern, key) pair its covering patterns give it, so a workgroup can run
// its queries through the keys of every covering pattern in turn and write
// final rows. Positions are grouped by residue mod L = lcm(r) inside windows
// of W = gcd(w') positions: every pattern covers all or none of a group (its
// r divides L, and its segments start at multiples of W), and a window lies
// inside one segment of every pattern. A workgroup takes up to
// 32 kOnePassWaves positions (rows m of the group at t0 + L m) of one
// (batch, head, window, residue) group.
constexpr int kOnePassWaves = 4;  // waves (32 group rows each) per one-pass workgroup

struct OnePassArgs {
  const void* q;
  const void* k;
  const void* v;
  void* out;
  float* lse;
  int64_t B;
  int64_t N;
  int32_t H;
  int32_t np;
  float sl2;     // softmax scale * log2(e)
  int32_t L;     // lcm of the dilation rates
  int32_t W;     // gcd of the effective segment lengths
  int32_t nblk;  // workgroups per (window, residue): ceil(ceil(W / L) / (32 kOnePassWaves))
  int64_t nwin;  // N / W
  PatDev pat[kMaxPat];  // caller's order
};

struct MergeArgs {
  void* out;
  float* lse;
  const float* ws;
  int64_t B;
  int64_t N;
  int32_t H;
  int32_t np;
  PatDev pat[kMaxPat];  // caller's order (the order of the merge's sums)
  // Row-enumerating launch (every position gathered by some pattern): the
  // patterns are ranked by dilation (rank[i] of pat[i]); a row with two or
  // more covering patterns is merged by the thread that enumerates it as a
  // gathered row of its second covering pattern in rank order. Set by the
  // launcher.
  int32_t rank[kMaxPat];
  int32_t nenum;                   // enumerated patterns
  int32_t enum_pat[kMaxPat];       // their indices into pat
  uint32_t enum_blk[kMaxPat + 1];  // first block of each
  FastDiv enum_head_div[kMaxPat];  // division by nseg * lmax (slots per head)
  FastDiv enum_lmax_div[kMaxPat];  // division by lmax
};

// Host side of the tile order: the group size and the divisors the device
// decode below uses, for a pattern with `ntile` tiles per unit in a
// launch's order. Groups hold 4 units; the last pattern's group is larger,
// up to what fills an XCD's 4 MiB L2 with the units' key and value rows
// (4 to 16 units), so that the XCD's list ends with its shortest tiles
// without sending more units' rows through the L2 at once than it holds.
inline void set_tile_divisors(PatDev* p, int32_t ntile, bool last) {
  p->ntile = ntile;
  int32_t g = 4;
  if (last) {
    const int64_t unit_bytes = (int64_t)p->lmax * kDh * 2 * 2;  // bf16 K and V rows
    const int64_t fit = ((int64_t)4 << 20) / (unit_bytes > 0 ? unit_bytes : 1);
    g = (int32_t)(fit < 4 ? 4 : fit > 16 ? 16 : fit);
  }
  p->group = g;
  p->nseg_div = make_fastdiv((uint32_t)p->nseg);
  p->g_div = make_fastdiv((uint32_t)g);
  p->grp_div = make_fastdiv((uint32_t)g * (uint32_t)ntile);
}

#if defined(__HIPCC__)
// a / b for a < 2^22 and b >= 1: the float reciprocal's quotient is off by
// at most one there, and one correction each way makes it exact.
__device__ inline uint32_t udiv_small(uint32_t a, uint32_t b) {
  uint32_t q = (uint32_t)((float)a * __builtin_amdgcn_rcpf((float)b));
  const int32_t r = (int32_t)(a - q * b);
  if (r < 0) --q;
  else if ((uint32_t)r >= b) ++q;
  return q;
}

// Block id -> (pattern, unit, tile rank) of the launch order described at
// AttnArgs: ids are dealt to the XCDs round-robin (id mod kXcds); each XCD
// gets its share of every pattern's units (patterns sorted by tiles per
// unit) and walks them in groups (PatDev::group units), the group's
// heaviest tiles first. Returns false for the
// padding ids of XCDs whose list is shorter than the longest one. All
// quantities are below 2^31 (the host keeps the grid so), so the decode is
// 32-bit: shifts, multiply-high divisions by divisors the host prepared
// (set_tile_divisors) and small float-reciprocal divisions. `rank` is the
// tile's position in its unit's heaviest-first order; `unit` is
// ((b * H) + h) * nseg + seg.
template <class Args>
__device__ inline bool decode_order(const Args& a, uint32_t id, int32_t* pat, uint32_t* unit,
                                    uint32_t* rank) {
  static_assert(kXcds == 8, "XCD decode written for 8 XCDs");
  const uint32_t x = id & 7u;
  uint32_t slot = id >> 3;
  for (int p = 0; p < a.np; ++p) {
    const PatDev& P = a.pat[p];
    const uint32_t u0 = (uint32_t)a.unit_start[p];
    const uint32_t units = (uint32_t)a.unit_start[p + 1] - u0;
    const uint32_t extra = (x - u0) & 7u;  // this XCD's first unit is u0 + extra
    const uint32_t cnt = extra < units ? (units - extra + 7u) >> 3 : 0u;
    const uint32_t nt = (uint32_t)P.ntile;
    const uint32_t ntot = cnt * nt;
    if (slot < ntot) {
      // groups of G units; the last one holds the remaining cnt mod G
      const uint32_t G = (uint32_t)P.group;
      const uint32_t gfull = fdiv(cnt, P.g_div);
      uint32_t gi = fdiv(slot, P.grp_div), gsz = G;
      if (gi >= gfull) {
        gi = gfull;
        gsz = cnt - G * gfull;
      }
      const uint32_t r0 = slot - gi * G * nt;  // below G * ntile < 2^21
      const uint32_t k = udiv_small(r0, gsz);
      *pat = p;
      *unit = extra + (G * gi + (r0 - k * gsz)) * 8u;
      *rank = k;
      return true;
    }
    slot -= ntot;
  }
  return false;
}
#endif

// ---------------------------------------------------------------- index maps

// Offset of head h inside every segment of a pattern with dilation r.
__host__ __device__ inline int32_t head_offset(int32_t h, int32_t r) { return h % r; }

// Rows a head with offset off gathers from one segment of length wp.
__host__ __device__ inline int32_t rows_gathered(int64_t wp, int32_t off, int32_t r) {
  return off < wp ? (int32_t)((wp - off + r - 1) / r) : 0;
}

// Sequence position of gathered row m of segment s.
__host__ __device__ inline int64_t gathered_pos(int64_t s, int64_t wp, int32_t off, int32_t r,
                                                int64_t m) {
  return s * wp + off + m * (int64_t)r;
}

// Inverse of gathered_pos for one head: s * lmax + m if position t is a
// gathered row, else -1. Positions are below 2^31.
__host__ __device__ inline int64_t compact_index(uint32_t t, const PatDev& p, int32_t off) {
  const uint32_t s = fdiv(t, p.wp_div);
  const int32_t rel = (int32_t)(t - s * p.wp_div.d) - off;
  if (rel < 0) return -1;
  const uint32_t m = fdiv((uint32_t)rel, p.r_div);
  if ((uint32_t)rel != m * (uint32_t)p.r) return -1;
  return (int64_t)s * p.lmax + m;
}

}  // namespace da
