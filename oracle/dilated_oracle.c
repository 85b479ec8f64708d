/*
 * Dilated-attention forward pass: plain CPU oracle.
 *
 * TEST INFRASTRUCTURE ONLY. This is the slow, obviously correct reference
 * that the GPU library is checked against. Only the test suite, the smoke
 * check and the benchmark's CPU-baseline leg load it. The product library
 * never links, imports or calls it, and the two share no code, headers,
 * tables or helpers.
 *
 * What it computes, with the passage each step follows:
 *
 *  1. Segments. A pattern (w, r) cuts the sequence of N tokens into
 *     consecutive segments of w tokens and attention stays inside a segment
 *     ("LONGNET: Scaling Transformer to 1 billion tokens" blog, section
 *     "LongNet's attention allocation principle"; "LongNet论文精读" page,
 *     section "Dilated Attention的工作原理", step 1).
 *  2. Dilation. Inside a segment only every r-th token takes part ("skip one
 *     token" for r = 2: blog, same section; 精读 page, step 2), and each head
 *     starts at its own offset (blog, paragraph on the multi-head mechanism;
 *     dakule.com news page, section "如何做到？", multi-head paragraph).
 *  3. Dense softmax attention among the gathered tokens of one segment
 *     ("sub-dot products": blog, same section; 精读 page, step 3).
 *  4. Results go back to their original positions (精读 page, step 4).
 *  5. Several patterns are mixed (blog: "a series of attention patterns";
 *     dakule.com page, section "如何做到？"). Their combination rule is not
 *     printed on the pages; see reading R1 below.
 *
 * Readings taken where the pages leave a step open (each one is also listed
 * in the design notes):
 *  R1 merge: the patterns covering a row are combined with weights
 *     proportional to each pattern's softmax denominator, i.e.
 *     out = sum_i exp(lse_i - LSE) * O_i with LSE = logsumexp_i(lse_i).
 *     This equals one softmax over the multiset union of all keys the row
 *     sees. PARITY UNPINNED against the original paper's text (absent from
 *     the pages); pinned internally by the brute-force union softmax.
 *  R2 head offset: head h (0-based) uses offset h mod r.
 *  R3 w not a multiple of r: the gathered positions are off + m*r < w, so a
 *     head gathers L = ceil((w - off) / r) rows and L can differ by head.
 *  R4 w larger than N: the segment length becomes min(w, N); N must be a
 *     multiple of it (the caller checks; this oracle asserts it).
 *  R5 causal masking is over the gathered order, which is the original order
 *     because the gathered positions increase; a row sees itself.
 *  R6 rows that a pattern does not gather get nothing from that pattern;
 *     a row no pattern gathers has out = 0 and lse = -inf.
 *  R7 scale: scores are scale * q.k with scale = 1/sqrt(Dh) unless given.
 *  R8 inputs stored as bf16 are widened exactly; all arithmetic is in the
 *     precision this file is built for (double, or float for the f32 copy).
 *
 * Two independent derivations of which keys a row sees:
 *  - orc_fwd_*  walks patterns -> segments -> the arithmetic progression of
 *    gathered positions (steps 1-4), then merges per row (step 5);
 *  - orc_rows_* walks single rows and finds covering patterns and keys by a
 *    membership test over the segment, never building the progression.
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>
#ifdef _OPENMP
#include <omp.h>
#endif

typedef struct {
  int32_t w;
  int32_t r;
} orc_pattern;

enum { ORC_IN_F64 = 0, ORC_IN_F32 = 1, ORC_IN_BF16 = 2 };

enum {
  ORC_OK = 0,
  ORC_ERR_ARG = -1,
  ORC_ERR_SHAPE = -2,
  ORC_ERR_NOMEM = -3,
};

/* Exact widening of one stored input element. bf16 is the upper half of an
 * IEEE single, so shifting its bits up by 16 gives the same value. */
static double orc_load(const void* p, int dtype, int64_t i) {
  if (dtype == ORC_IN_F64) return ((const double*)p)[i];
  if (dtype == ORC_IN_F32) return (double)((const float*)p)[i];
  uint32_t u = ((uint32_t)((const uint16_t*)p)[i]) << 16;
  float f;
  memcpy(&f, &u, sizeof f);
  return (double)f;
}

static void orc_set_threads(int nthreads) {
#ifdef _OPENMP
  if (nthreads > 0) omp_set_num_threads(nthreads);
#else
  (void)nthreads;
#endif
}

int orc_max_threads(void) {
#ifdef _OPENMP
  return omp_get_max_threads();
#else
  return 1;
#endif
}

/* Step 1-2 geometry of one pattern for one head.
 * wp   : effective segment length min(w, N)            (R4)
 * nseg : number of segments N / wp
 * off  : first gathered position inside a segment      (R2)
 * L    : gathered rows per segment, ceil((wp-off)/r)   (R3) */
int orc_geometry(int64_t N, int32_t w, int32_t r, int32_t h, int64_t* wp, int64_t* nseg,
                 int64_t* off, int64_t* L) {
  if (N < 1 || w < 1 || r < 1 || h < 0) return ORC_ERR_ARG;
  int64_t wpv = (int64_t)w < N ? (int64_t)w : N;
  if (N % wpv != 0) return ORC_ERR_SHAPE;
  int64_t o = (int64_t)(h % r);
  int64_t l = o < wpv ? (wpv - o + r - 1) / r : 0;
  if (wp) *wp = wpv;
  if (nseg) *nseg = N / wpv;
  if (off) *off = o;
  if (L) *L = l;
  return ORC_OK;
}

/* The gather list of one pattern for head h: for every segment s in order,
 * the positions s*wp + off + m*r for m = 0..L-1. Returns the count written,
 * or a negative code if cap is too small. */
int64_t orc_gather_map(int64_t N, int32_t w, int32_t r, int32_t h, int64_t* out, int64_t cap) {
  int64_t wp, nseg, off, L;
  int rc = orc_geometry(N, w, r, h, &wp, &nseg, &off, &L);
  if (rc) return rc;
  if (nseg * L > cap) return ORC_ERR_ARG;
  int64_t n = 0;
  for (int64_t s = 0; s < nseg; ++s)
    for (int64_t m = 0; m < L; ++m) out[n++] = s * wp + off + m * r;
  return n;
}

/* Coverage of position t by pattern (w, r) for head h, found by membership
 * (used by the row-wise oracle): t is gathered when its distance from its
 * segment's start is off modulo r. */
static int orc_covers(int64_t N, int32_t w, int32_t r, int32_t h, int64_t t, int64_t* seg0,
                      int64_t* wp_out) {
  int64_t wp = (int64_t)w < N ? (int64_t)w : N;
  int64_t s0 = (t / wp) * wp;
  if (seg0) *seg0 = s0;
  if (wp_out) *wp_out = wp;
  return ((t - s0) % r) == (int64_t)(h % r);
}

/* The definition body is written once and instantiated for double and
 * float; the f32 copy exists only to show the scale of fp32 rounding. */
#define REAL double
#define RSFX f64
#define REXP exp
#define RLOG log
#include "oracle_core.inc"
#undef REAL
#undef RSFX
#undef REXP
#undef RLOG

#define REAL float
#define RSFX f32
#define REXP expf
#define RLOG logf
#include "oracle_core.inc"
#undef REAL
#undef RSFX
#undef REXP
#undef RLOG
