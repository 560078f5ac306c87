/*
 * ep_oracle.c -- plain, slow CPU oracle for MoE expert-parallel token
 * dispatch, combine, combine backward, the static-shape planner and the
 * duplicated-expert gradient reduce.
 *
 * TEST INFRASTRUCTURE ONLY.  Only the tests, the smoke check and the
 * benchmark's CPU-baseline leg load this library.  It shares no code, header,
 * table or helper with the GPU library: both sides see only the seeded input
 * arrays.
 *
 * Pages the method is described on (cited by title and section):
 *   [MoonEP] Open Source For You, "Moonshot AI's MoonEP ..." news article:
 *            paragraph 3 (predictable per-rank workload, GPU planner choosing
 *            redundant experts from the current router output), paragraph 4
 *            (rows go straight to expert-grouped positions, static shapes),
 *            paragraph 5 (prefetch slots bounded by E/R in training, a
 *            small fixed number in inference with overflow read from the
 *            owner directly; a dedicated reduce buffer folds
 *            duplicated-expert gradients into the owner's gradients).
 *   [NCCLEP] listing of the NCCL EP paper (arXiv 2603.13606): abstract
 *            (LL and HT modes), Table II (combine gathers expert outputs and
 *            reduces them to the original token order), Table III (LL: 3D
 *            expert-major output; HT: 2D output with token counts), Table IV
 *            (tensor roles: tokens, top-k indices, top-k weights, FP8
 *            scales), Figures 3-5.
 *   [ULMoE]  "Ultra-Large MoE Models: Open-Source Evolution and Heterogeneous
 *            Inference Adaptation", section 3.1 (top-k routing operator;
 *            grouped GEMM over the tokens grouped by expert), section 4.1
 *            (experts split over devices in contiguous blocks).
 *            The expert FFN around the grouped GEMM is not spelled out
 *            there; READING: the gated SiLU (SwiGLU) of the large MoE
 *            models those pages discuss, see orc_swiglu.
 * Every point those pages leave open is marked READING below and listed in
 * the design notes of the repository.
 *
 * Floating point.  Sums of products are carried in double and rounded once
 * to the output type (bf16 or fp32, round-to-nearest-even).  The FP8 code of
 * an element is decided in fp32, the precision the GPU kernel decides it in.
 * The duplicated-expert reduce adds in double in replica order and rounds
 * once to fp32.  Build with -ffp-contract=off so that no multiply-add is
 * fused behind the code's back.
 *
 * Parity status: every function below is pinned by CPU tests against
 * library routines, closed forms, brute force or hand-worked cases, except
 * that the planner's *rule* is a reading (the pages give its contract, not
 * its algorithm); its outputs are pinned by invariants and hand-worked cases.
 */
#include <float.h>
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>
#ifdef _OPENMP
#include <omp.h>
#endif

#define ORC_FLAG_INDEX_RANGE 1u
#define ORC_FLAG_CAPACITY 2u
#define ORC_FLAG_SLOT_BUDGET 4u

#define ORC_LAYOUT_LL 0
#define ORC_LAYOUT_HT 1
#define ORC_LAYOUT_STATIC 2

/* ------------------------------------------------------------------------ */
/* threads (timing only; results do not depend on the thread count)          */
/* ------------------------------------------------------------------------ */

void orc_set_threads(int n) {
#ifdef _OPENMP
  if (n > 0) omp_set_num_threads(n);
#else
  (void)n;
#endif
}

int orc_get_threads(void) {
#ifdef _OPENMP
  return omp_get_max_threads();
#else
  return 1;
#endif
}

/* ------------------------------------------------------------------------ */
/* number formats                                                            */
/* ------------------------------------------------------------------------ */

/* bf16 bit pattern -> value (exact: bf16 is the top half of an fp32). */
double orc_bf16_to_double(uint16_t b) {
  uint32_t u = (uint32_t)b << 16;
  float f;
  memcpy(&f, &u, sizeof f);
  return (double)f;
}

/* Nearest bf16 to v, ties to even (bf16: 1 sign, 8 exponent bits with
 * fp32's bias, 8 significant bits).  The value is rounded to a multiple of
 * the bf16 spacing of its binade with rint (ties to even in the default
 * rounding mode); the result then has at most 8 significant bits and is
 * exactly representable in fp32, whose top 16 bits are the bf16 pattern. */
uint16_t orc_bf16_from_double(double v) {
  if (isnan(v)) return 0x7FC0;
  uint16_t sign = signbit(v) ? 0x8000 : 0;
  double a = fabs(v);
  if (a == 0.0) return sign;
  if (isinf(a)) return (uint16_t)(sign | 0x7F80);
  int ex;
  frexp(a, &ex);              /* a in [2^(ex-1), 2^ex) */
  int e = ex - 1;
  if (e < -126) e = -126;     /* subnormal range: spacing stays 2^-133 */
  double ulp = ldexp(1.0, e - 7);
  double r = rint(a / ulp) * ulp;
  if (r >= ldexp(1.0, 128)) return (uint16_t)(sign | 0x7F80);
  float f = (float)r;         /* exact */
  uint32_t u;
  memcpy(&u, &f, sizeof u);
  return (uint16_t)(sign | (uint16_t)(u >> 16));
}

/* Nearest OCP FP8 E4M3 ("e4m3fn": bias 7, 4 significant bits, largest
 * finite 448, no infinities, S.1111.111 is NaN) to v, ties to even.
 * Magnitudes above 448 saturate to 448 (callers clamp first anyway). */
uint8_t orc_e4m3_from_float(float v) {
  if (isnan(v)) return 0x7F;
  uint8_t sign = signbit(v) ? 0x80 : 0;
  double a = fabs((double)v);
  if (a > 448.0) a = 448.0;
  if (a == 0.0) return sign;
  int ex;
  frexp(a, &ex);
  int e = ex - 1;
  if (e < -6) e = -6;         /* subnormals: 0.mmm x 2^-6, spacing 2^-9 */
  double ulp = ldexp(1.0, e - 3);
  double r = rint(a / ulp) * ulp;
  int code;
  if (r < ldexp(1.0, -6)) {
    code = (int)(r / ldexp(1.0, -9));
  } else {
    int ex2;
    frexp(r, &ex2);
    int E = ex2 - 1;          /* r in [2^E, 2^(E+1)) */
    int mant = (int)((r / ldexp(1.0, E) - 1.0) * 8.0);
    code = ((E + 7) << 3) | mant;
  }
  return (uint8_t)(sign | (uint8_t)code);
}

double orc_e4m3_to_double(uint8_t c) {
  int s = c >> 7, E = (c >> 3) & 15, m = c & 7;
  if (E == 15 && m == 7) return NAN;
  double mag = (E == 0) ? ldexp((double)m, -9) : ldexp(1.0 + m / 8.0, E - 7);
  return s ? -mag : mag;
}

/* ------------------------------------------------------------------------ */
/* layout: per-expert counts, offsets, stable positions, destination rows    */
/* ------------------------------------------------------------------------ */

/*
 * [NCCLEP] Table III and Figures 3-4: dispatch turns the 2D token input into
 * an expert-grouped output.  Entry f = t*k + j (token t, choice j) goes to
 * expert idx[f].
 *   counts[e]  = number of entries routed to e            (HT "token counts")
 *   offsets[e] = counts[0] + ... + counts[e-1], offsets[E] = total
 *   pos[f]     = number of earlier entries f' < f with idx[f'] == idx[f]
 * READING: rows inside one expert keep the flat entry order (the pages fix
 * no order; this one matches "back to the original token order").
 * READING: idx == -1 means "no expert" and is skipped; any other value
 * outside [0, E) is skipped too and raises the INDEX_RANGE flag.
 * Returns the flags.
 */
uint32_t orc_layout(int32_t T, int32_t k, int32_t E, const int32_t *idx,
                    int32_t *counts, int32_t *offsets, int32_t *pos) {
  uint32_t flags = 0;
  int64_t n = (int64_t)T * k;
  for (int32_t e = 0; e < E; ++e) counts[e] = 0;
  for (int64_t f = 0; f < n; ++f) {
    int32_t e = idx[f];
    if (e < 0 || e >= E) {
      if (e != -1) flags |= ORC_FLAG_INDEX_RANGE;
      pos[f] = -1;
      continue;
    }
    pos[f] = counts[e];       /* entries of e seen so far = earlier entries of e */
    counts[e] += 1;
  }
  offsets[0] = 0;
  for (int32_t e = 0; e < E; ++e) offsets[e + 1] = offsets[e] + counts[e];
  return flags;
}

/*
 * Destination row of every entry for the two layouts of [NCCLEP] Table III.
 *   HT (2D concatenated rows, [T*k, H]):  dst = offsets[e] + pos
 *   LL (3D expert-major, [E, cap, H]):    dst = e*cap + pos   if pos < cap
 * READING: an LL entry with pos >= cap is dropped (dst = -1, CAPACITY flag).
 * Skipped entries get dst = -1.  Returns the flags.
 */
uint32_t orc_dst_ht_ll(int32_t T, int32_t k, int32_t layout, int32_t cap,
                       const int32_t *idx, const int32_t *pos,
                       const int32_t *offsets, int32_t *dst) {
  uint32_t flags = 0;
  int64_t n = (int64_t)T * k;
  for (int64_t f = 0; f < n; ++f) {
    if (pos[f] < 0) { dst[f] = -1; continue; }
    int32_t e = idx[f];
    if (layout == ORC_LAYOUT_HT) {
      dst[f] = offsets[e] + pos[f];
    } else {
      if (pos[f] < cap) {
        dst[f] = e * cap + pos[f];
      } else {
        dst[f] = -1;
        flags |= ORC_FLAG_CAPACITY;
      }
    }
  }
  return flags;
}

/* ------------------------------------------------------------------------ */
/* static-shape planner                                                      */
/* ------------------------------------------------------------------------ */

/*
 * [MoonEP] paragraphs 3-5: every rank gets a workload of known size whatever
 * the routing; a GPU planner picks redundant experts from the current router
 * output; a training rank has at most E/R prefetch slots for the duplicates.
 * [ULMoE] section 4.1: experts are split over ranks in contiguous blocks, so
 * expert e lives on rank e / m with m = E / R.
 *
 * READING (the pages give the contract, not the rule).  With N routed rows:
 *  1. every rank takes target(r) = floor(N/R) + (r < N mod R) rows, in a
 *     buffer of C >= ceil(N/R) rows (C is the static shape, from T*k);
 *  2. home(r) = rows of rank r's own experts;
 *  3. a rank with home(r) > target(r) is a donor with excess X: it walks its
 *     experts hottest first (count descending, id ascending) and sheds
 *     min(count, remaining X) rows of each, always the *last* positions of
 *     that expert; keep[e] = count - shed;
 *  4. the shed pieces form one sequence (donor rank ascending, then walk
 *     order); the ranks with home(r) < target(r) form the receivers
 *     (ascending), each wanting target - home rows;
 *  5. both sequences are laid end to end and intersected: each non-empty
 *     overlap of a piece and a receiver is one segment -- a run of
 *     consecutive positions of one expert placed on one receiver;
 *  6. a rank's rows are its own experts' kept rows in expert order, then the
 *     segments it received in sequence order;
 *  7. a receiver numbers the distinct experts it received 0, 1, ... in
 *     sequence order; the first S of them get its replica slots.  A segment
 *     past the S-th has no slot: in training mode (slot_mode 0) that raises
 *     SLOT_BUDGET, since a training rank reserves slots for all of its
 *     duplicates; in inference mode (slot_mode 1) it is the overflow case
 *     of [MoonEP] paragraph 5 -- a small fixed number of slots, the rest
 *     read from the owner's weights directly -- and raises nothing.  The
 *     plan's rows are the same in both modes.
 *
 * Outputs (arrays sized by the caller):
 *   keep[E], native_row[E]     kept rows of e and their first row in home rank
 *   seg_first[E], seg_count[E] e's segments in the segment list
 *   seg[(E+R)*5]               (expert, rank, pos_begin, len, row_begin)
 *   *n_seg                     number of segments
 *   load[R]                    rows used on each rank (= target)
 *   replica[R*S]               expert in each replica slot, -1 if empty
 *   seg_slot[E+R]              slot of each segment on its rank, -1 if none
 *   *flags                     ORed with SLOT_BUDGET if a receiver needs > S
 *                              in training mode
 * Returns 0, or -1 if the arguments are inconsistent (E % R != 0, C too small,
 * negative counts).
 */
int32_t orc_plan(int32_t E, int32_t R, int32_t S, int32_t C, int32_t slot_mode,
                 const int32_t *counts, int32_t *keep, int32_t *native_row,
                 int32_t *seg_first, int32_t *seg_count, int32_t *seg, int32_t *n_seg,
                 int32_t *load, int32_t *replica, int32_t *seg_slot, uint32_t *flags) {
  if (E <= 0 || R <= 0 || E % R != 0 || S < 0 || slot_mode < 0 || slot_mode > 1) return -1;
  int32_t m = E / R;
  int64_t N = 0;
  for (int32_t e = 0; e < E; ++e) {
    if (counts[e] < 0) return -1;
    N += counts[e];
  }
  if ((int64_t)C * R < N) return -1;

  int64_t *target = (int64_t *)malloc(sizeof(int64_t) * R);
  int64_t *home = (int64_t *)malloc(sizeof(int64_t) * R);
  int32_t *shed = (int32_t *)malloc(sizeof(int32_t) * E);
  int32_t *order = (int32_t *)malloc(sizeof(int32_t) * (m > 0 ? m : 1));
  /* pieces: expert, first shed position, length, start in the spill sequence */
  int32_t *pc_e = (int32_t *)malloc(sizeof(int32_t) * E);
  int64_t *pc_start = (int64_t *)malloc(sizeof(int64_t) * E);
  int32_t *pc_len = (int32_t *)malloc(sizeof(int32_t) * E);
  int32_t n_pc = 0;

  /* step 1, 2 */
  for (int32_t r = 0; r < R; ++r) {
    target[r] = N / R + (r < N % R ? 1 : 0);
    home[r] = 0;
    for (int32_t e = r * m; e < (r + 1) * m; ++e) home[r] += counts[e];
  }
  /* step 3, 4: donors shed tail rows, hottest expert first */
  int64_t spill = 0;
  for (int32_t e = 0; e < E; ++e) shed[e] = 0;
  for (int32_t r = 0; r < R; ++r) {
    if (home[r] <= target[r]) continue;
    int64_t X = home[r] - target[r];
    for (int32_t i = 0; i < m; ++i) order[i] = r * m + i;
    /* insertion sort: count descending, id ascending */
    for (int32_t i = 1; i < m; ++i) {
      int32_t v = order[i], j = i - 1;
      while (j >= 0 && (counts[order[j]] < counts[v] ||
                        (counts[order[j]] == counts[v] && order[j] > v))) {
        order[j + 1] = order[j];
        --j;
      }
      order[j + 1] = v;
    }
    for (int32_t i = 0; i < m && X > 0; ++i) {
      int32_t e = order[i];
      int32_t s = counts[e] < X ? counts[e] : (int32_t)X;
      if (s <= 0) continue;
      shed[e] = s;
      X -= s;
      pc_e[n_pc] = e;
      pc_start[n_pc] = spill;
      pc_len[n_pc] = s;
      spill += s;
      ++n_pc;
    }
  }
  for (int32_t e = 0; e < E; ++e) keep[e] = counts[e] - shed[e];

  /* step 6 (own rows): kept rows of each rank in expert order */
  for (int32_t r = 0; r < R; ++r) {
    int32_t row = 0;
    for (int32_t e = r * m; e < (r + 1) * m; ++e) {
      native_row[e] = row;
      row += keep[e];
    }
  }

  /* step 5: intersect the spill sequence with the receivers' deficits */
  for (int32_t e = 0; e < E; ++e) { seg_first[e] = 0; seg_count[e] = 0; }
  for (int32_t i = 0; i < R * S; ++i) replica[i] = -1;
  int32_t ns = 0;
  int32_t pi = 0;
  int64_t want_start = 0;
  int32_t *slots_used = (int32_t *)calloc((size_t)R, sizeof(int32_t));
  for (int32_t r = 0; r < R; ++r) {
    if (home[r] >= target[r]) continue;
    int64_t d_lo = want_start, d_hi = want_start + (target[r] - home[r]);
    want_start = d_hi;
    while (pi < n_pc) {
      int64_t p_lo = pc_start[pi], p_hi = pc_start[pi] + pc_len[pi];
      int64_t a = p_lo > d_lo ? p_lo : d_lo;
      int64_t b = p_hi < d_hi ? p_hi : d_hi;
      if (a < b) {
        int32_t e = pc_e[pi];
        if (seg_count[e] == 0) seg_first[e] = ns;
        seg_count[e] += 1;
        seg[ns * 5 + 0] = e;
        seg[ns * 5 + 1] = r;
        seg[ns * 5 + 2] = keep[e] + (int32_t)(a - p_lo);     /* position in e */
        seg[ns * 5 + 3] = (int32_t)(b - a);
        seg[ns * 5 + 4] = (int32_t)(home[r] + (a - d_lo));  /* row in rank r */
        /* step 7: replica slot on the receiver */
        if (slots_used[r] < S) {
          replica[r * S + slots_used[r]] = e;
          seg_slot[ns] = slots_used[r];
        } else {
          seg_slot[ns] = -1;
          if (slot_mode == 0) *flags |= ORC_FLAG_SLOT_BUDGET;
        }
        slots_used[r] += 1;
        ++ns;
      }
      if (p_hi <= d_hi) ++pi;   /* piece used up: next piece */
      if (d_hi <= p_hi) break;  /* receiver full: next receiver */
    }
  }
  *n_seg = ns;
  for (int32_t r = 0; r < R; ++r) load[r] = (int32_t)target[r];

  free(slots_used);
  free(target); free(home); free(shed); free(order);
  free(pc_e); free(pc_start); free(pc_len);
  return 0;
}

/*
 * Replica-weight prefetch, [MoonEP] paragraphs 3 and 5: the planner picks
 * redundant experts from the current routing and their weights are
 * prefetched into dedicated slots of the receiving rank; the weights of
 * each expert projection sit contiguously.  Definition: for every slot
 * (r, s) with replica[r*S+s] = e >= 0, slot (r, s) becomes a byte copy of
 * expert e's row of `weights`; empty slots are left as they are.
 *   weights  [E][row_bytes]      each expert's projection, contiguous
 *   slots    [R*S][row_bytes]    the ranks' prefetch slots
 * Returns -1 if a slot names an expert outside [0, E), else 0.
 */
int32_t orc_prefetch(int32_t E, int32_t R, int32_t S, int64_t row_bytes,
                     const int32_t *replica, const uint8_t *weights, uint8_t *slots) {
  for (int64_t i = 0; i < (int64_t)R * S; ++i) {
    const int32_t e = replica[i];
    if (e < 0) continue;
    if (e >= E) return -1;
    for (int64_t b = 0; b < row_bytes; ++b) slots[i * row_bytes + b] = weights[(int64_t)e * row_bytes + b];
  }
  return 0;
}

/*
 * Destination row of every entry in the static layout [R, C, H]: a kept
 * position lands in its home rank after the rows of lower experts of that
 * rank; a shed position lands in the segment that covers it.
 */
void orc_dst_static(int32_t T, int32_t k, int32_t E, int32_t R, int32_t C,
                    const int32_t *idx, const int32_t *pos, const int32_t *keep,
                    const int32_t *native_row, const int32_t *seg_first,
                    const int32_t *seg_count, const int32_t *seg, int32_t *dst) {
  int32_t m = E / R;
  int64_t n = (int64_t)T * k;
  for (int64_t f = 0; f < n; ++f) {
    dst[f] = -1;
    if (pos[f] < 0) continue;
    int32_t e = idx[f], p = pos[f];
    if (p < keep[e]) {
      dst[f] = (e / m) * C + native_row[e] + p;
      continue;
    }
    for (int32_t s = seg_first[e]; s < seg_first[e] + seg_count[e]; ++s) {
      int32_t pb = seg[s * 5 + 2], len = seg[s * 5 + 3];
      if (p >= pb && p < pb + len) {
        dst[f] = seg[s * 5 + 1] * C + seg[s * 5 + 4] + (p - pb);
        break;
      }
    }
  }
}

/* ------------------------------------------------------------------------ */
/* dispatch                                                                  */
/* ------------------------------------------------------------------------ */

/*
 * [MoonEP] paragraph 4 / [NCCLEP] Table III: token rows are written straight
 * into their expert-grouped destination rows.  recv[dst[f], :] = x[t, :],
 * bit for bit.  Rows no entry maps to are left untouched.
 */
void orc_dispatch(int32_t T, int32_t k, int32_t H, const uint16_t *x,
                  const int32_t *dst, uint16_t *recv) {
  int64_t t;
#pragma omp parallel for schedule(static)
  for (t = 0; t < T; ++t) {
    for (int32_t j = 0; j < k; ++j) {
      int32_t d = dst[t * k + j];
      if (d < 0) continue;
      for (int32_t h = 0; h < H; ++h) recv[(int64_t)d * H + h] = x[(int64_t)t * H + h];
    }
  }
}

/*
 * Receive-side metadata per row ([NCCLEP] Table V: dispatch also hands back
 * the received indices and weights): the source entry, the expert and the
 * router weight of each row; -1 / -1 / 0 for rows no entry maps to.
 */
void orc_recv_meta(int32_t T, int32_t k, int64_t rows, const int32_t *idx,
                   const float *w, const int32_t *dst, int32_t *recv_src,
                   int32_t *recv_idx, float *recv_w) {
  for (int64_t r = 0; r < rows; ++r) {
    recv_src[r] = -1;
    if (recv_idx) recv_idx[r] = -1;
    if (recv_w) recv_w[r] = 0.0f;
  }
  for (int64_t f = 0; f < (int64_t)T * k; ++f) {
    int32_t d = dst[f];
    if (d < 0) continue;
    recv_src[d] = (int32_t)f;
    if (recv_idx) recv_idx[d] = idx[f];
    if (recv_w && w) recv_w[d] = w[f];
  }
}

/*
 * FP8 quantisation of one token row, per block of 128 channels ([NCCLEP]
 * Table IV names FP8 scales as a tensor role; the recipe is a READING):
 *   amax = max |x| over the block (exact),  s = amax / 448 in fp32 (1 if 0),
 *   q    = E4M3(clamp(x / s, -448, 448)),   x / s an fp32 division.
 * The dequantised value is q * s.
 *
 * Power-of-two scales (READING, a second format a group can choose; the
 * pages fix none): s is the smallest power of two not below the fp32
 * quotient amax / 448, and not below 2^-126, the smallest normal fp32, so
 * that its exponent is a valid 8-bit block exponent; 1 if amax is 0.  The
 * codes are decided as above; x / s is then a power-of-two division.
 */
static float pow2_scale(float amax) {
  if (amax == 0.0f) return 1.0f;
  float t = amax / 448.0f;
  int e;
  float m = frexpf(t, &e); /* t = m * 2^e, 0.5 <= m < 1 */
  float s = (m == 0.5f) ? t : ldexpf(1.0f, e);
  return s < FLT_MIN ? FLT_MIN : s;
}

static void quantize_row(int32_t H, const uint16_t *x, uint8_t *q, float *scale, int pow2) {
  for (int32_t b = 0; b < H / 128; ++b) {
    float amax = 0.0f;
    for (int32_t c = 0; c < 128; ++c) {
      float v = (float)fabs(orc_bf16_to_double(x[b * 128 + c]));
      if (v > amax) amax = v;
    }
    float s = pow2 ? pow2_scale(amax) : (amax == 0.0f) ? 1.0f : amax / 448.0f;
    scale[b] = s;
    for (int32_t c = 0; c < 128; ++c) {
      float v = (float)orc_bf16_to_double(x[b * 128 + c]) / s;
      if (v > 448.0f) v = 448.0f;
      if (v < -448.0f) v = -448.0f;
      q[b * 128 + c] = orc_e4m3_from_float(v);
    }
  }
}

void orc_quantize_row_fp8(int32_t H, const uint16_t *x, uint8_t *q, float *scale) {
  quantize_row(H, x, q, scale, 0);
}

void orc_quantize_row_fp8_pow2(int32_t H, const uint16_t *x, uint8_t *q, float *scale) {
  quantize_row(H, x, q, scale, 1);
}

static void dispatch_fp8(int32_t T, int32_t k, int32_t H, const uint16_t *x, const int32_t *dst,
                         uint8_t *recv_q, float *recv_scale, int pow2) {
  int32_t nb = H / 128;
  int64_t t;
#pragma omp parallel for schedule(static)
  for (t = 0; t < T; ++t) {
    uint8_t *q = (uint8_t *)malloc((size_t)H);
    float *s = (float *)malloc(sizeof(float) * (size_t)(nb > 0 ? nb : 1));
    quantize_row(H, x + (int64_t)t * H, q, s, pow2);
    for (int32_t j = 0; j < k; ++j) {
      int32_t d = dst[t * k + j];
      if (d < 0) continue;
      memcpy(recv_q + (int64_t)d * H, q, (size_t)H);
      memcpy(recv_scale + (int64_t)d * nb, s, sizeof(float) * (size_t)nb);
    }
    free(q);
    free(s);
  }
}

void orc_dispatch_fp8(int32_t T, int32_t k, int32_t H, const uint16_t *x,
                      const int32_t *dst, uint8_t *recv_q, float *recv_scale) {
  dispatch_fp8(T, k, H, x, dst, recv_q, recv_scale, 0);
}

void orc_dispatch_fp8_pow2(int32_t T, int32_t k, int32_t H, const uint16_t *x,
                           const int32_t *dst, uint8_t *recv_q, float *recv_scale) {
  dispatch_fp8(T, k, H, x, dst, recv_q, recv_scale, 1);
}

/* ------------------------------------------------------------------------ */
/* combine and backward                                                      */
/* ------------------------------------------------------------------------ */

/*
 * [NCCLEP] Table II / Table III: combine gathers the expert outputs of each
 * token and reduces them back to the token's place:
 *   y[t, h] = sum_j w[t, j] * out[dst[t, j], h]      (j ascending, dst >= 0)
 * in double, rounded once to bf16 (out_fp32 == 0) or fp32 (out_fp32 != 0).
 * w == NULL means every weight is 1: this is the backward of dispatch, the
 * sum of the gradient rows of a token's copies.
 */
void orc_combine(int32_t T, int32_t k, int32_t H, const uint16_t *rows,
                 const int32_t *dst, const float *w, int32_t out_fp32, void *y) {
  int64_t t;
#pragma omp parallel for schedule(static)
  for (t = 0; t < T; ++t) {
    for (int32_t h = 0; h < H; ++h) {
      double acc = 0.0;
      for (int32_t j = 0; j < k; ++j) {
        int32_t d = dst[t * k + j];
        if (d < 0) continue;
        double wj = w ? (double)w[t * k + j] : 1.0;
        acc += wj * orc_bf16_to_double(rows[(int64_t)d * H + h]);
      }
      if (out_fp32) ((float *)y)[(int64_t)t * H + h] = (float)acc;
      else ((uint16_t *)y)[(int64_t)t * H + h] = orc_bf16_from_double(acc);
    }
  }
}

/*
 * Backward of combine ([NCCLEP] Figure 5: the routing state of the forward
 * pass is reused by the backward pass).  With y[t] = sum_j w[t,j] out[dst]:
 *   grad_out[dst[t,j], h] = bf16( w[t,j] * gy[t,h] )   (one rounding)
 *   grad_w[t, j]          = sum_h gy[t,h] * out[dst[t,j], h]   (fp32 result)
 * Skipped entries: grad_w = 0 and no row written.
 */
void orc_combine_bwd(int32_t T, int32_t k, int32_t H, const uint16_t *gy,
                     const uint16_t *out, const int32_t *dst, const float *w,
                     uint16_t *grad_out, float *grad_w) {
  int64_t t;
#pragma omp parallel for schedule(static)
  for (t = 0; t < T; ++t) {
    for (int32_t j = 0; j < k; ++j) {
      int32_t d = dst[t * k + j];
      if (d < 0) { grad_w[t * k + j] = 0.0f; continue; }
      double wj = (double)w[t * k + j];
      double dot = 0.0;
      for (int32_t h = 0; h < H; ++h) {
        double g = orc_bf16_to_double(gy[(int64_t)t * H + h]);
        grad_out[(int64_t)d * H + h] = orc_bf16_from_double(wj * g);
        dot += g * orc_bf16_to_double(out[(int64_t)d * H + h]);
      }
      grad_w[t * k + j] = (float)dot;
    }
  }
}

/* ------------------------------------------------------------------------ */
/* duplicated-expert gradient reduce                                         */
/* ------------------------------------------------------------------------ */

/*
 * [MoonEP] paragraph 5: gradients of duplicated experts pass through a
 * reduce buffer and are accumulated into the owner's parameter gradients.
 *   owner[e, p] <- fp32( owner[e, p] + sum_{i : rep_e[i] == e} rep[i, p] )
 * with the sum taken in double in replica order i = 0, 1, ... and rounded
 * once; rep_e[i] == -1 skips replica i.  Owners no replica names are left
 * untouched.
 */
void orc_dup_reduce(int32_t n, int64_t P, const uint16_t *rep, const int32_t *rep_e,
                    int32_t E, float *owner) {
  for (int32_t e = 0; e < E; ++e) {
    int any = 0;
    for (int32_t i = 0; i < n; ++i) any |= (rep_e[i] == e);
    if (!any) continue;
    int64_t p;
#pragma omp parallel for schedule(static)
    for (p = 0; p < P; ++p) {
      double acc = (double)owner[(int64_t)e * P + p];
      for (int32_t i = 0; i < n; ++i)
        if (rep_e[i] == e) acc += orc_bf16_to_double(rep[(int64_t)i * P + p]);
      owner[(int64_t)e * P + p] = (float)acc;
    }
  }
}

/* ------------------------------------------------------------------------ */
/* grouped GEMM of the experts                                               */
/* ------------------------------------------------------------------------ */

/*
 * [ULMoE] section 3.1: the core of the expert computation is a grouped GEMM
 * -- the tokens, grouped by expert, are multiplied by their expert's weights,
 * one irregularly sized matrix product per expert.  [NCCLEP] Figure 2 puts
 * the expert FFN between dispatch and combine, on the dispatched rows.
 * READING: one product per group of consecutive receive rows that share a
 * weight matrix; the weights of each expert are one [N][K] matrix (a linear
 * layer's layout, K contiguous), and a prefetch slot holds a copy of one.
 * Definition, for every group g = (row0, rows, widx), row i < rows and
 * column n < N:
 *   Y[row0 + i][n] = bf16( sum_{c < K} X[row0 + i][c] * W[widx][n][c] )
 * with the sum taken in double (each bf16 x bf16 product is exact there)
 * and rounded once, to nearest even.  Rows of Y that no group covers are
 * left unchanged.
 *   groups  [ngroups][3]   row0, rows, widx
 *   X       [.][K] bf16    the receive buffer
 *   W       [.][N][K] bf16 the table of weight matrices
 *   Y       [.][N] bf16
 */
void orc_grouped_gemm(int32_t ngroups, const int32_t *groups, int32_t K, int32_t N,
                      const uint16_t *X, const uint16_t *W, uint16_t *Y) {
  for (int32_t g = 0; g < ngroups; ++g) {
    const int64_t row0 = groups[g * 3 + 0], rows = groups[g * 3 + 1], widx = groups[g * 3 + 2];
    const uint16_t *Wg = W + widx * (int64_t)N * K;
    int64_t i;
#pragma omp parallel for schedule(static)
    for (i = 0; i < rows; ++i) {
      const uint16_t *x = X + (row0 + i) * K;
      for (int32_t n = 0; n < N; ++n) {
        const uint16_t *w = Wg + (int64_t)n * K;
        double acc = 0.0;
        for (int32_t c = 0; c < K; ++c) acc += orc_bf16_to_double(x[c]) * orc_bf16_to_double(w[c]);
        Y[(row0 + i) * N + n] = orc_bf16_from_double(acc);
      }
    }
  }
}

/*
 * The same grouped GEMM on FP8 operands: the receive rows as ep_dispatch's
 * FP8 path leaves them ([NCCLEP] Table IV: e4m3 codes with one fp32 scale
 * per 128 channels) and weights in the same format, one scale per output
 * row n and 128-wide block of K.  READING: a code stands for code * scale,
 * so, for every group g = (row0, rows, widx), row i and column n,
 *   Y[row0 + i][n] = bf16( sum_b SX[row0 + i][b] * SW[widx][n][b] *
 *                          sum_{c in block b} X[row0 + i][c] * W[widx][n][c] )
 * with the codes decoded exactly (OCP e4m3), all sums in double and one
 * rounding to bf16.
 *   X  [.][K] e4m3, SX [.][K/128] fp32; W [.][N][K] e4m3, SW [.][N][K/128] fp32
 */
void orc_grouped_gemm_fp8(int32_t ngroups, const int32_t *groups, int32_t K, int32_t N,
                          const uint8_t *X, const float *SX, const uint8_t *W, const float *SW,
                          uint16_t *Y) {
  const int32_t nb = K / 128;
  for (int32_t g = 0; g < ngroups; ++g) {
    const int64_t row0 = groups[g * 3 + 0], rows = groups[g * 3 + 1], widx = groups[g * 3 + 2];
    int64_t i;
#pragma omp parallel for schedule(static)
    for (i = 0; i < rows; ++i) {
      const uint8_t *x = X + (row0 + i) * K;
      const float *sx = SX + (row0 + i) * nb;
      for (int32_t n = 0; n < N; ++n) {
        const uint8_t *w = W + (widx * N + n) * (int64_t)K;
        const float *sw = SW + (widx * N + n) * (int64_t)nb;
        double acc = 0.0;
        for (int32_t b = 0; b < nb; ++b) {
          double part = 0.0;
          for (int32_t c = b * 128; c < (b + 1) * 128; ++c)
            part += orc_e4m3_to_double(x[c]) * orc_e4m3_to_double(w[c]);
          acc += (double)sx[b] * (double)sw[b] * part;
        }
        Y[(row0 + i) * N + n] = orc_bf16_from_double(acc);
      }
    }
  }
}

/* ------------------------------------------------------------------------ */
/* top-k routing                                                             */
/* ------------------------------------------------------------------------ */

/*
 * [UL-MoE] sections 2.1 and 3.1: the gate's scores pick a few experts per
 * token (top-k); section 3.2 names a fused top-k + routing operator.  The
 * NCCL EP listing's Table IV takes the chosen indices and weights as inputs.
 * READING: experts in descending logit order, equal logits to the lower
 * expert id, choice j = 0 the largest; weights are the softmax over the k
 * chosen logits.  With fewer than k experts the extra choices are -1 with
 * weight 0.  Logits must be finite.
 * Selection: k rounds, each taking the largest logit not yet taken (first
 * index wins a tie).  Softmax in double, rounded once to fp32.
 */
void orc_route(int32_t T, int32_t E, int32_t k, const float *logits, int32_t *idx, float *w) {
  int64_t t;
#pragma omp parallel for schedule(static)
  for (t = 0; t < T; ++t) {
    const float *l = logits + t * E;
    char *taken = (char *)calloc((size_t)(E > 0 ? E : 1), 1);
    double *z = (double *)calloc((size_t)(k > 0 ? k : 1), sizeof(double));
    int32_t n = 0;
    for (int32_t j = 0; j < k; ++j) {
      int32_t best = -1;
      for (int32_t e = 0; e < E; ++e) {
        if (taken[e]) continue;
        if (best < 0 || l[e] > l[best]) best = e;
      }
      idx[t * k + j] = best;
      if (best >= 0) {
        taken[best] = 1;
        ++n;
      }
    }
    double m = n > 0 ? (double)l[idx[t * k]] : 0.0;
    double sum = 0.0;
    for (int32_t j = 0; j < n; ++j) {
      z[j] = exp((double)l[idx[t * k + j]] - m);
      sum += z[j];
    }
    for (int32_t j = 0; j < k; ++j) w[t * k + j] = j < n ? (float)(z[j] / sum) : 0.0f;
    free(z);
    free(taken);
  }
}

/* The activation between the expert FFN's two grouped GEMMs ([ULMoE]
 * section 3.1 names the grouped GEMM as the core of the expert computation;
 * READING: the activation is SwiGLU, and the first GEMM's weight rows come
 * interleaved, row 2j the gate projection of output j and row 2j + 1 its up
 * projection, so each output column's pair is adjacent).  For h of
 * [rows, 2I] bf16 and every j < I:
 *   out[r, j] = bf16( silu(g) * u ),  g = h[r, 2j],  u = h[r, 2j + 1],
 *   silu(g) = g / (1 + e^(-g)),
 * in double, rounded once to nearest even. */
void orc_swiglu(int64_t rows, int32_t I, const uint16_t *h, uint16_t *out) {
  for (int64_t r = 0; r < rows; ++r)
    for (int32_t j = 0; j < I; ++j) {
      const double g = orc_bf16_to_double(h[r * 2 * I + 2 * j]);
      const double u = orc_bf16_to_double(h[r * 2 * I + 2 * j + 1]);
      const double silu = g / (1.0 + exp(-g));
      out[r * I + j] = orc_bf16_from_double(silu * u);
    }
}
