/*
 * CPU ORACLE for the routed-MoE layer step.  TEST INFRASTRUCTURE ONLY:
 * only the test suite, the smoke check and the benchmark's CPU-baseline leg
 * load this library.  The HIP library shares no code with it.
 *
 * Plain C11, no intrinsics, built with -O2 -ffp-contract=off -fno-fast-math
 * (OpenMP only across independent output rows; results do not depend on the
 * thread count).  Each function follows one step of the method as the pages
 * state it, with the readings below where the pages are silent.
 *
 * Sources (cited by page title and section):
 *  [HN]  "Show HN: 遅いコンピュータで GLM 5.2 を実行する" (ja.news.hada.io),
 *        section 実装済みの主な機能 (implemented features): DeepSeek-V3-style
 *        sigmoid router with noaux_tc, routed_scaling_factor and a shared
 *        expert; integer-dot kernels taking Q8_0-style int8 activations;
 *        int8 / packed int4 / packed int2 weights with per-row scales,
 *        dequantised on use; batch-union MoE reading each distinct expert once
 *        per batch and applying it to every position routed to it.
 *  [HN-S] same page, section ディスクストリーミングベースの MoE 実行方式:
 *        ~19 MB per int4 expert.
 *  [HN-R] same page, section モデルのダウンロードと実行 (download and run),
 *        its list of options: an adaptive expert top-p (value 0.7 given)
 *        that cuts expert reads by 30-40%; [HN-B] section コミュニティ
 *        ベンチマーク: that option gave 1.6x end to end.
 *  [DT-M] devtrends page below, section "Modèles supportés": one supported
 *        model reads native MXFP4 weights directly from its shards.
 *  [DT]  "Comment exécuter un réseau de neurones de 744 milliards de
 *        paramètres sur un ordinateur ordinaire" (devtrends.cc), section
 *        "Comment fonctionne le moteur": requests for the same expert are
 *        merged; an expert's three matrices are read together.
 *
 * Readings where the pages are silent, one per point:
 *  R1 noaux_tc: the per-expert correction bias enters expert *selection*
 *     only; routing weights use the unbiased sigmoid score.
 *  R2 group score = sum of the two largest biased scores in the group; the
 *     topk_group best groups are kept, the others excluded.
 *  R3 ties: lower group index, then lower expert index; idx is listed in
 *     rank order (biased score descending, index ascending).
 *  R4 weights: w_k = (s_k / S) * routed_scaling, S = s_0 + s_1 + ... in
 *     rank order, all fp32.
 *  R5 router arithmetic is fp32 in one fixed order (dot_canon, exp_canon
 *     below) so that the selected indices are a function of the inputs alone.
 *  R6 Q8_0: blocks of 32, fp32 scale d = amax/127, q = roundf(x * (1/d))
 *     (half away from zero), clamped to [-127,127]; amax = 0 gives d = 0, q = 0.
 *  R7 the SwiGLU hidden vector h is Q8_0-quantised before the down matrix
 *     (the integer-dot kernels take int8 activations).
 *  R8 expert FFN = down( silu(gate x) * (up x) ), silu(z) = z / (1 + e^-z).
 *  R9 combine: y = shared + sum_k w_k * expert_k (shared expert weight 1).
 *  R10 packed codes: int4 element 2j in the low nibble of byte j, 2j+1 in the
 *     high nibble; int2 element 4j+i in bits 2i..2i+1; two's complement.
 *  R16 MXFP4 experts (wbits code ORACLE_MXFP4 below): the OCP microscaling
 *     format -- FP4 E2M1 elements (sign bit, 2-bit exponent with bias 1,
 *     1-bit mantissa: magnitudes 0, 0.5, 1, 1.5, 2, 3, 4, 6), two per byte
 *     (element 2j in the low nibble), and one E8M0 scale byte s per 32
 *     consecutive elements of a row, value 2^(s-127); no per-row scale.
 *     Record: gate codes [I][H/2], up codes [I][H/2], down codes [H][I/2],
 *     then the scale bytes gate [I][H/32], up [I][H/32], down [H][I/32].
 *     Activations stay Q8_0 (the engine's integer kernels take them), so a
 *     row is sum_b 2^(s_b-127) * d_b * sum_k fp4(c_k) q_k; the integer block
 *     dot reported for it is P2 = sum_k (2 fp4(c_k)) q_k (2 fp4 is an integer).
 *  R18 FP8 experts (wbits code ORACLE_FP8 below): one page says a supported
 *     model runs on fp4/fp8 weights, another that the engine's converter
 *     dequantises FP8 checkpoints with one scale per 128x128 block.  The
 *     format is therefore OCP FP8 E4M3 ("FN": sign bit, 4-bit exponent with
 *     bias 7, 3-bit mantissa, no infinities; codes 0x7F and 0xFF are NaN and
 *     not valid weights; normal value (1 + m/8) 2^(e-7), subnormal (e = 0)
 *     m 2^-9, largest 448), one byte per element, and one fp32 scale per
 *     128x128 block of each matrix.  Record: gate codes [I][H], up [I][H],
 *     down [H][I], then the fp32 block scales gate [I/128][H/128], up
 *     [I/128][H/128], down [H/128][I/128].  Activations stay Q8_0, so a row r
 *     is sum_b S[r/128][b/4] * d_b * sum_k fp8(c_k) q_k over the 32-blocks
 *     b; since 512 fp8 is an integer (|512 fp8| <= 229376), the block dot
 *     P9 = sum_k (512 fp8(c_k)) q_k is exact in int32 and is what the debug
 *     dumps report (the row is then sum_b S * d_b * P9_b / 512).
 *  R15 adaptive expert top-p (p in (0,1); 0 or 1 = off): after the top-K
 *     selection, keep the shortest prefix of the rank order whose unbiased
 *     scores, summed left to right in fp32, reach p * S (fp32 product; S as
 *     in R4); the kept weights are renormalised over that prefix,
 *     w_k = (s_k / S_kept) * routed_scaling; a dropped rank has idx -1 and
 *     w 0 and is read by no later step.
 *
 *  R17 per-row activation scales (declared format beside Q8_0; activation
 *     block "row", ablk = -1 below): the pages' integer kernels take Q8_0
 *     blocks of 32; this second format applies the R6 rule to a whole
 *     activation row at once -- one fp32 scale d = amax(row)/127 per token
 *     row of x (H values) and per (token, expert) row of h (I values),
 *     q = clamp(roundf(x * (1/d)), -127, 127) -- so that an output row is
 *     scale_r * d * P with P the exact integer dot over the whole row
 *     (|P| <= 6144 * 128 * 127 < 2^31 at the real shape).  Integer codes
 *     only (MXFP4 keeps its per-32 weight scales, hence Q8_0 blocks).
 *
 * Precision: router fp32 (R5); Q8_0 decisions fp32; block dots exact in
 * int64 (checked to fit int32); the float epilogues in fp64, rounded to fp32.
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

#define QBLK 32

/* ---------------------------------------------------------------- codes */

#define ORACLE_MXFP4 (-4)
#define ORACLE_FP8 (-8)
#define F8BLK 128

/* R16: value of an FP4 E2M1 code (0..15) and of an E8M0 scale byte. */
double oracle_fp4_value(int code) {
  static const double mag[8] = {0.0, 0.5, 1.0, 1.5, 2.0, 3.0, 4.0, 6.0};
  const double v = mag[code & 7];
  return (code & 8) ? -v : v;
}
double oracle_e8m0_value(int s) { return ldexp(1.0, s - 127); }

/* R18: value of an FP8 E4M3 code (0..255); NaN for 0x7F and 0xFF. */
double oracle_fp8_value(int code) {
  const int e = (code >> 3) & 15, m = code & 7;
  double v;
  if (e == 15 && m == 7) return NAN;
  if (e == 0) v = ldexp((double)m, -9);
  else v = ldexp(1.0 + m / 8.0, e - 7);
  return (code & 0x80) ? -v : v;
}

/* Element k of a packed weight row (R10; MXFP4: the raw 4-bit code, R16). */
int oracle_code(const uint8_t *row, int wbits, int k) {
  if (wbits == ORACLE_FP8) return row[k];  /* the raw byte, R18 */
  if (wbits == ORACLE_MXFP4) {
    int b = row[k / 2];
    return (k % 2 == 0) ? (b & 0xF) : ((b >> 4) & 0xF);
  }
  if (wbits == 4) {
    int b = row[k / 2];
    int v = (k % 2 == 0) ? (b & 0xF) : ((b >> 4) & 0xF);
    return v >= 8 ? v - 16 : v;
  }
  if (wbits == 2) {
    int b = row[k / 4];
    int v = (b >> (2 * (k % 4))) & 0x3;
    return v >= 2 ? v - 4 : v;
  }
  if (wbits == 8) return (int)(int8_t)row[k];
  return 0;
}

/* All n codes of a packed row. */
void oracle_unpack(const uint8_t *row, int wbits, int n, int8_t *out) {
  for (int k = 0; k < n; k++) out[k] = (int8_t)oracle_code(row, wbits, k);
}

/* Inverse of oracle_code over a row of n codes (used by the pins). */
int oracle_pack(const int8_t *codes, int n, int wbits, uint8_t *out) {
  if (wbits == ORACLE_MXFP4) {  /* raw 4-bit codes 0..15, element 2j low */
    if (n % 2) return -1;
    for (int j = 0; j < n / 2; j++) {
      if (codes[2 * j] < 0 || codes[2 * j] > 15 || codes[2 * j + 1] < 0 || codes[2 * j + 1] > 15)
        return -1;
      out[j] = (uint8_t)(codes[2 * j] | (codes[2 * j + 1] << 4));
    }
    return 0;
  }
  if (wbits == 8 || wbits == ORACLE_FP8) {  /* one byte per code (FP8: the raw byte) */
    for (int k = 0; k < n; k++) out[k] = (uint8_t)codes[k];
    return 0;
  }
  if (wbits != 4 && wbits != 2) return -1;
  const int per = 8 / wbits;
  if (n % per) return -1;
  for (int j = 0; j < n / per; j++) {
    unsigned b = 0;
    for (int i = 0; i < per; i++) {
      int c = codes[j * per + i];
      int lo = (wbits == 4) ? -8 : -2, hi = (wbits == 4) ? 7 : 1;
      if (c < lo || c > hi) return -1;
      unsigned field = (unsigned)(c < 0 ? c + (1 << wbits) : c);
      b |= field << (wbits * i);
    }
    out[j] = (uint8_t)b;
  }
  return 0;
}

/* ---------------------------------------------------------------- Q8_0 */

/* Activation block length of format ablk on a row of n values: Q8_0 (32)
 * or the whole row (R17, ablk = -1); 0 if ablk is neither. */
static int act_len(int ablk, int n) { return ablk == -1 ? n : ablk == QBLK ? QBLK : 0; }

/* R6 (and R17 with ablk = -1), [HN] integer-dot item: rows x rows of n
 * floats -> int8 codes and one fp32 scale per block of the format:
 * d = amax/127, q = clamp(roundf(x * (1/d)), -127, 127). */
int oracle_quant_act(const float *x, int64_t rows, int n, int ablk, int8_t *q, float *d) {
  const int B = act_len(ablk, n);
  if (B <= 0 || n % B) return -1;
  const int nb = n / B;
  for (int64_t r = 0; r < rows; r++) {
    for (int b = 0; b < nb; b++) {
      const float *xb = x + r * n + (int64_t)b * B;
      float amax = 0.0f;
      for (int k = 0; k < B; k++) amax = fmaxf(amax, fabsf(xb[k]));
      float dd = amax / 127.0f;
      float id = (dd != 0.0f) ? 1.0f / dd : 0.0f;
      d[r * nb + b] = dd;
      for (int k = 0; k < B; k++) {
        float v = roundf(xb[k] * id);
        if (v > 127.0f) v = 127.0f;
        if (v < -127.0f) v = -127.0f;
        q[r * n + (int64_t)b * B + k] = (int8_t)v;
      }
    }
  }
  return 0;
}

/* R6: Q8_0, blocks of 32. */
int oracle_q8_0(const float *x, int64_t rows, int n, int8_t *q, float *d) {
  return oracle_quant_act(x, rows, n, QBLK, q, d);
}

/* ---------------------------------------------------------------- router */

/* R5: fixed-order fp32 dot product.  k runs in consecutive chunks of 64;
 * each chunk is an fma chain in increasing k starting from 0, and the chunk
 * partials are added left to right. */
float oracle_dot_canon(const float *a, const float *b, int n) {
  float total = 0.0f;
  for (int c = 0; c < n; c += 64) {
    float part = 0.0f;
    for (int k = c; k < c + 64 && k < n; k++) part = fmaf(a[k], b[k], part);
    total = (c == 0) ? part : total + part;
  }
  return total;
}

/* R5: e^y in fp32 from IEEE basic operations: Cody–Waite reduction by ln 2
 * split into a 24-bit-exact high part and a low part, then the degree-7
 * Taylor polynomial of e^r by Horner with fma, then scaling by 2^n. */
float oracle_exp_canon(float y) {
  const float LOG2E = 1.44269502f;           /* fp32(log2 e)            */
  const float LN2_HI = 0.693145751953125f;   /* ln 2 cut to 16 bits     */
  const float LN2_LO = 1.42860677e-06f;      /* fp32(ln 2 - LN2_HI)     */
  if (y > 87.0f) y = 87.0f;
  if (y < -87.0f) y = -87.0f;
  float n = rintf(y * LOG2E);
  float r = fmaf(-n, LN2_HI, y);
  r = fmaf(-n, LN2_LO, r);
  /* 1/k! rounded to fp32, k = 7 .. 0 */
  float p = 1.98412701e-04f;
  p = fmaf(p, r, 1.38888892e-03f);
  p = fmaf(p, r, 8.33333377e-03f);
  p = fmaf(p, r, 4.16666679e-02f);
  p = fmaf(p, r, 1.66666672e-01f);
  p = fmaf(p, r, 0.5f);
  p = fmaf(p, r, 1.0f);
  p = fmaf(p, r, 1.0f);
  return ldexpf(p, (int)n);
}

float oracle_sigmoid_canon(float l) { return 1.0f / (1.0f + oracle_exp_canon(-l)); }

/* [HN] router item, R1/R5: s = sigmoid(x . W_r[e]), sb = s + bias[e]. */
void oracle_router_scores(int T, int H, int E, const float *x, const float *wr,
                          const float *bias, float *s, float *sb) {
#pragma omp parallel for collapse(2) schedule(static)
  for (int t = 0; t < T; t++)
    for (int e = 0; e < E; e++) {
      float l = oracle_dot_canon(x + (size_t)t * H, wr + (size_t)e * H, H);
      float v = oracle_sigmoid_canon(l);
      s[(size_t)t * E + e] = v;
      sb[(size_t)t * E + e] = v + bias[e];
    }
}

/* [HN] noaux_tc + routed_scaling_factor, R1-R4: group-limited top-k for one
 * token given its unbiased (s) and biased (sb) scores.  Selection is repeated
 * argmax with strict '>' scanning in increasing index, so equal values go to
 * the lower index.  margin (nullable) receives, in fp64, the gap between the
 * K-th and (K+1)-th selected candidate and between the TG-th and (TG+1)-th
 * group (a diagnostic of how close the decision was). */
int oracle_select_one(int E, int G, int TG, int K, float scale, const float *s,
                      const float *sb, int32_t *idx, float *w, double *margin) {
  const int gs = E / G;
  if (E % G || gs < 2 || TG < 1 || TG > G || K < 1 || K > TG * gs) return -1;
  float *gscore = (float *)malloc(sizeof(float) * G);
  char *kept = (char *)calloc(G, 1), *taken = (char *)calloc(E, 1);
  for (int g = 0; g < G; g++) {
    int i1 = -1, i2 = -1;
    for (int e = g * gs; e < (g + 1) * gs; e++)
      if (i1 < 0 || sb[e] > sb[i1]) i1 = e;
    for (int e = g * gs; e < (g + 1) * gs; e++)
      if (e != i1 && (i2 < 0 || sb[e] > sb[i2])) i2 = e;
    gscore[g] = sb[i1] + sb[i2];
  }
  float last_group = 0.0f;
  for (int j = 0; j < TG; j++) {
    int best = -1;
    for (int g = 0; g < G; g++)
      if (!kept[g] && (best < 0 || gscore[g] > gscore[best])) best = g;
    kept[best] = 1;
    last_group = gscore[best];
  }
  float last_pick = 0.0f;
  for (int k = 0; k < K; k++) {
    int best = -1;
    for (int e = 0; e < E; e++)
      if (kept[e / gs] && !taken[e] && (best < 0 || sb[e] > sb[best])) best = e;
    taken[best] = 1;
    idx[k] = best;
    last_pick = sb[best];
  }
  float S = 0.0f;
  for (int k = 0; k < K; k++) S = S + s[idx[k]];
  for (int k = 0; k < K; k++) w[k] = (s[idx[k]] / S) * scale;
  if (margin) {
    double next_pick = -INFINITY, next_group = -INFINITY;
    for (int e = 0; e < E; e++)
      if (kept[e / gs] && !taken[e] && sb[e] > next_pick) next_pick = sb[e];
    for (int g = 0; g < G; g++)
      if (!kept[g] && gscore[g] > next_group) next_group = gscore[g];
    margin[0] = (double)last_pick - next_pick;
    margin[1] = (double)last_group - next_group;
  }
  free(gscore);
  free(kept);
  free(taken);
  return 0;
}

int oracle_select(int T, int E, int G, int TG, int K, float scale, const float *s,
                  const float *sb, int32_t *idx, float *w, double *margin) {
  for (int t = 0; t < T; t++) {
    int rc = oracle_select_one(E, G, TG, K, scale, s + (size_t)t * E, sb + (size_t)t * E,
                               idx + (size_t)t * K, w + (size_t)t * K,
                               margin ? margin + 2 * (size_t)t : NULL);
    if (rc) return rc;
  }
  return 0;
}

/* [HN-R] adaptive expert top-p, reading R15, applied in place to one
 * token's rank-ordered selection (idx, w) given its unbiased scores s[E].
 * Returns the number of experts kept. */
int oracle_top_p_one(int K, int E, float p, float scale, const float *s, int32_t *idx,
                     float *w) {
  if (!(p > 0.0f && p < 1.0f)) return K;  /* off: the plain top-K */
  float S = 0.0f;
  for (int k = 0; k < K; k++) {
    if (idx[k] < 0 || idx[k] >= E) return -1;
    S = S + s[idx[k]];
  }
  const float thr = p * S;
  float cum = 0.0f;
  int kept = K;
  for (int k = 0; k < K; k++) {
    cum = cum + s[idx[k]];
    if (cum >= thr) {
      kept = k + 1;
      break;
    }
  }
  float S_kept = 0.0f;
  for (int k = 0; k < kept; k++) S_kept = S_kept + s[idx[k]];
  for (int k = 0; k < K; k++) {
    if (k < kept) {
      w[k] = (s[idx[k]] / S_kept) * scale;
    } else {
      idx[k] = -1;
      w[k] = 0.0f;
    }
  }
  return kept;
}

int oracle_top_p(int T, int K, int E, float p, float scale, const float *s, int32_t *idx,
                 float *w, int32_t *kept) {
  for (int t = 0; t < T; t++) {
    int r = oracle_top_p_one(K, E, p, scale, s + (size_t)t * E, idx + (size_t)t * K,
                             w + (size_t)t * K);
    if (r < 0) return -1;
    if (kept) kept[t] = r;
  }
  return 0;
}

int oracle_route(int T, int H, int E, int G, int TG, int K, float scale, const float *x,
                 const float *wr, const float *bias, int32_t *idx, float *w,
                 double *margin) {
  if (H % 64) return -1;
  float *s = (float *)malloc(sizeof(float) * (size_t)T * E);
  float *sb = (float *)malloc(sizeof(float) * (size_t)T * E);
  oracle_router_scores(T, H, E, x, wr, bias, s, sb);
  int rc = oracle_select(T, E, G, TG, K, scale, s, sb, idx, w, margin);
  free(s);
  free(sb);
  return rc;
}

/* ---------------------------------------------------------------- grouping */

/* [HN] batch-union item, [DT] merged requests: token slots (slot = t*K + k)
 * grouped by expert with a counting sort in slot order, so each expert's list
 * is in increasing token order; active = experts with at least one slot,
 * ascending, padded with -1.  A slot dropped by top-p (idx -1, R15) joins no
 * list: inv = -1, and perm holds the offsets[E] kept slots followed by -1. */
int oracle_group(int T, int K, int E, const int32_t *idx, int32_t *counts,
                 int32_t *offsets, int32_t *perm, int32_t *inv, int32_t *active,
                 int32_t *n_active) {
  const int n = T * K;
  for (int e = 0; e < E; e++) counts[e] = 0;
  for (int i = 0; i < n; i++) {
    if (idx[i] == -1) continue;
    if (idx[i] < 0 || idx[i] >= E) return -1;
    counts[idx[i]]++;
  }
  offsets[0] = 0;
  for (int e = 0; e < E; e++) offsets[e + 1] = offsets[e] + counts[e];
  int32_t *cursor = (int32_t *)malloc(sizeof(int32_t) * (E > 0 ? E : 1));
  for (int e = 0; e < E; e++) cursor[e] = offsets[e];
  for (int i = offsets[E]; i < n; i++) perm[i] = -1;
  for (int i = 0; i < n; i++) {
    if (idx[i] == -1) {
      inv[i] = -1;
      continue;
    }
    int p = cursor[idx[i]]++;
    perm[p] = i;
    inv[i] = p;
  }
  free(cursor);
  int na = 0;
  for (int e = 0; e < E; e++)
    if (counts[e] > 0) active[na++] = e;
  for (int e = na; e < E; e++) active[e] = -1;
  *n_active = na;
  return 0;
}

/* ---------------------------------------------------------------- expert FFN */

/* Exact integer dot of each activation block (32 values, or the whole row
 * for R17) of a packed weight row with int8 activations ([HN] integer-dot
 * and quantisation items). */
int oracle_act_dots(const uint8_t *row, int wbits, const int8_t *q, int n, int ablk,
                    int32_t *out) {
  const int B = act_len(ablk, n);
  if (B <= 0 || n % B || ((wbits == ORACLE_MXFP4 || wbits == ORACLE_FP8) && B != QBLK)) return -1;
  for (int b = 0; b < n / B; b++) {
    int64_t acc = 0;
    for (int k = b * B; k < (b + 1) * B; k++) {
      const int c = oracle_code(row, wbits, k);
      if (wbits == ORACLE_FP8 && isnan(oracle_fp8_value(c))) return -1;
      const int64_t wv = wbits == ORACLE_MXFP4 ? (int64_t)(2.0 * oracle_fp4_value(c))
                         : wbits == ORACLE_FP8 ? (int64_t)(512.0 * oracle_fp8_value(c))
                                               : c;
      acc += wv * (int64_t)q[k];
    }
    if (acc > INT32_MAX || acc < INT32_MIN) return -1;
    out[b] = (int32_t)acc;
  }
  return 0;
}

int oracle_block_dots(const uint8_t *row, int wbits, const int8_t *q, int n, int32_t *out) {
  return oracle_act_dots(row, wbits, q, n, QBLK, out);
}

size_t oracle_blob_bytes(int H, int I, int wbits) {
  if (wbits == ORACLE_FP8)  /* R18: byte codes, one fp32 scale per 128x128 block */
    return (size_t)3 * I * H + sizeof(float) * 3 * (size_t)(I / F8BLK) * (H / F8BLK);
  if (wbits == ORACLE_MXFP4)  /* R16: 4-bit codes, one scale byte per 32 */
    return ((size_t)2 * I * H + (size_t)H * I) / 2 + ((size_t)2 * I * H + (size_t)H * I) / QBLK;
  return ((size_t)2 * I * H + (size_t)H * I) * (size_t)wbits / 8 +
         sizeof(float) * ((size_t)2 * I + H);
}

typedef struct {
  const uint8_t *gate, *up, *down;
  const float *sg, *su, *sd;        /* per-row scales (integer codes) */
  const uint8_t *bg, *bu, *bd;      /* per-block E8M0 scales (MXFP4) */
  const float *fg, *fu, *fd;        /* 128x128 block scales (FP8) */
  size_t gate_row, down_row;
} blob_view;

static blob_view view_of(const uint8_t *blob, int H, int I, int wbits) {
  blob_view v;
  const int bits = wbits == ORACLE_MXFP4 ? 4 : wbits == ORACLE_FP8 ? 8 : wbits;
  v.gate_row = (size_t)H * bits / 8;
  v.down_row = (size_t)I * bits / 8;
  v.gate = blob;
  v.up = blob + (size_t)I * v.gate_row;
  v.down = blob + 2 * (size_t)I * v.gate_row;
  const uint8_t *tail = v.down + (size_t)H * v.down_row;
  v.sg = v.su = v.sd = NULL;
  v.bg = v.bu = v.bd = NULL;
  v.fg = v.fu = v.fd = NULL;
  if (wbits == ORACLE_FP8) {
    const float *sc = (const float *)tail;
    const size_t nb = (size_t)(I / F8BLK) * (H / F8BLK);
    v.fg = sc;
    v.fu = sc + nb;
    v.fd = sc + 2 * nb;
  } else if (wbits == ORACLE_MXFP4) {
    v.bg = tail;
    v.bu = tail + (size_t)I * (H / QBLK);
    v.bd = tail + 2 * (size_t)I * (H / QBLK);
  } else {
    const float *sc = (const float *)tail;
    v.sg = sc;
    v.su = sc + I;
    v.sd = sc + 2 * I;
  }
  return v;
}

/* fp64 value of one output row (dequantise on use), activation blocks of
 * the format ablk (nb = n / block length of them): integer codes
 * scale_r * sum_b d_b * P_b; MXFP4 (bsc: the row's block scales, Q8_0 only)
 * sum_b 2^(s_b-127) * d_b * P2_b / 2. */
static double row_value(const uint8_t *row, int wbits, int ablk, float scale,
                        const uint8_t *bsc, const float *fsc, const int8_t *q, const float *d,
                        int n, int32_t *dots_out, int *err) {
  const int B = act_len(ablk, n);
  if (B <= 0) {
    *err = 1;
    return 0.0;
  }
  const int nb = n / B;
  int32_t P[QBLK * 16];
  int32_t *dots = dots_out;
  int32_t *tmp = NULL;
  if (!dots) {
    if (nb <= (int)(sizeof(P) / sizeof(P[0]))) dots = P;
    else dots = tmp = (int32_t *)malloc(sizeof(int32_t) * (size_t)nb);
  }
  if (oracle_act_dots(row, wbits, q, n, ablk, dots)) *err = 1;
  double acc = 0.0;
  if (bsc) {
    for (int b = 0; b < nb; b++)
      acc += oracle_e8m0_value(bsc[b]) * (double)d[b] * (0.5 * (double)dots[b]);
    free(tmp);
    return acc;
  }
  if (fsc) {  /* R18: the 128-block scale of each group of four 32-blocks */
    for (int b = 0; b < nb; b++)
      acc += (double)fsc[b / (F8BLK / QBLK)] * (double)d[b] * ((double)dots[b] / 512.0);
    free(tmp);
    return acc;
  }
  for (int b = 0; b < nb; b++) acc += (double)d[b] * (double)dots[b];
  free(tmp);
  return (double)scale * acc;
}

/* Gate and up projections plus SwiGLU for one token (R8), activations in
 * format ablk (Q8_0: 32; R17 rows: -1).  q, d: the token's activations (H
 * values; d one scale per block).  Outputs (each nullable): gate_dots and
 * up_dots [I][H/block] int32, g and u [I] fp64, h [I] fp32 =
 * fp32(silu(g) * u). */
int oracle_gate_up_act(const uint8_t *blob, int H, int I, int wbits, int ablk, const int8_t *q,
                       const float *d, int32_t *gate_dots, int32_t *up_dots, double *g_out,
                       double *u_out, float *h) {
  const int B = act_len(ablk, H);
  if (H % QBLK || I % QBLK || B <= 0) return -1;
  if (wbits == ORACLE_FP8 && (H % F8BLK || I % F8BLK)) return -1;
  blob_view v = view_of(blob, H, I, wbits);
  int err = 0;
#pragma omp parallel for schedule(static) reduction(| : err)
  for (int r = 0; r < I; r++) {
    int e1 = 0;
    const int mx = wbits == ORACLE_MXFP4, f8 = wbits == ORACLE_FP8;
    const size_t fo = (size_t)(r / F8BLK) * (H / F8BLK);  /* the row's 128-block scales */
    double g = row_value(v.gate + r * v.gate_row, wbits, ablk, mx || f8 ? 1.0f : v.sg[r],
                         mx ? v.bg + (size_t)r * (H / QBLK) : NULL, f8 ? v.fg + fo : NULL, q,
                         d, H, gate_dots ? gate_dots + (size_t)r * (H / B) : NULL, &e1);
    double u = row_value(v.up + r * v.gate_row, wbits, ablk, mx || f8 ? 1.0f : v.su[r],
                         mx ? v.bu + (size_t)r * (H / QBLK) : NULL, f8 ? v.fu + fo : NULL, q,
                         d, H, up_dots ? up_dots + (size_t)r * (H / B) : NULL, &e1);
    double silu = g / (1.0 + exp(-g));
    if (g_out) g_out[r] = g;
    if (u_out) u_out[r] = u;
    if (h) h[r] = (float)(silu * u);
    err |= e1;
  }
  return err ? -1 : 0;
}

int oracle_gate_up(const uint8_t *blob, int H, int I, int wbits, const int8_t *q,
                   const float *d, int32_t *gate_dots, int32_t *up_dots, double *g_out,
                   double *u_out, float *h) {
  return oracle_gate_up_act(blob, H, I, wbits, QBLK, q, d, gate_dots, up_dots, g_out, u_out, h);
}

/* Down projection for one token, activations (qh, dh: h of I values) in
 * format ablk.  Outputs (nullable): down_dots [H][I/block] int32, y [H]
 * fp32. */
int oracle_down_act(const uint8_t *blob, int H, int I, int wbits, int ablk, const int8_t *qh,
                    const float *dh, int32_t *down_dots, float *y) {
  const int B = act_len(ablk, I);
  if (H % QBLK || I % QBLK || B <= 0) return -1;
  if (wbits == ORACLE_FP8 && (H % F8BLK || I % F8BLK)) return -1;
  blob_view v = view_of(blob, H, I, wbits);
  int err = 0;
#pragma omp parallel for schedule(static) reduction(| : err)
  for (int j = 0; j < H; j++) {
    int e1 = 0;
    const int mx = wbits == ORACLE_MXFP4, f8 = wbits == ORACLE_FP8;
    const size_t fo = (size_t)(j / F8BLK) * (I / F8BLK);
    double val = row_value(v.down + j * v.down_row, wbits, ablk, mx || f8 ? 1.0f : v.sd[j],
                           mx ? v.bd + (size_t)j * (I / QBLK) : NULL, f8 ? v.fd + fo : NULL, qh,
                           dh, I, down_dots ? down_dots + (size_t)j * (I / B) : NULL, &e1);
    if (y) y[j] = (float)val;
    err |= e1;
  }
  return err ? -1 : 0;
}

int oracle_down(const uint8_t *blob, int H, int I, int wbits, const int8_t *qh,
                const float *dh, int32_t *down_dots, float *y) {
  return oracle_down_act(blob, H, I, wbits, QBLK, qh, dh, down_dots, y);
}

/* Whole expert for one token: gate/up, SwiGLU, quantisation of h in the same
 * activation format (R7, R17), down.  h, qh, dh nullable (intermediates for
 * inspection; dh has I/block entries); y [H] required. */
int oracle_expert_act(const uint8_t *blob, int H, int I, int wbits, int ablk, const int8_t *q,
                      const float *d, float *h_out, int8_t *qh_out, float *dh_out, float *y) {
  const int B = act_len(ablk, I);
  if (B <= 0) return -1;
  float *h = (float *)malloc(sizeof(float) * I);
  int8_t *qh = (int8_t *)malloc((size_t)I);
  float *dh = (float *)malloc(sizeof(float) * (I / B));
  int rc = oracle_gate_up_act(blob, H, I, wbits, ablk, q, d, NULL, NULL, NULL, NULL, h);
  if (!rc) rc = oracle_quant_act(h, 1, I, ablk, qh, dh);
  if (!rc) rc = oracle_down_act(blob, H, I, wbits, ablk, qh, dh, NULL, y);
  if (h_out) memcpy(h_out, h, sizeof(float) * I);
  if (qh_out) memcpy(qh_out, qh, (size_t)I);
  if (dh_out) memcpy(dh_out, dh, sizeof(float) * (I / B));
  free(h);
  free(qh);
  free(dh);
  return rc;
}

int oracle_expert(const uint8_t *blob, int H, int I, int wbits, const int8_t *q,
                  const float *d, float *h_out, int8_t *qh_out, float *dh_out, float *y) {
  return oracle_expert_act(blob, H, I, wbits, QBLK, q, d, h_out, qh_out, dh_out, y);
}

/* ---------------------------------------------------------------- combine */

/* R9, [HN] shared-expert item: y[t] = residual[t] + shared[t] + sum_k w[t,k] *
 * expert_out[t,k] (residual and shared nullable), in fp64 in rank order.
 * y_norm (nullable) = y / sqrt(mean(y^2) + eps) with unit gain (the norm that
 * feeds the next layer of a stack). */
void oracle_combine(int T, int H, int K, const float *expert_out, const float *w,
                    const float *shared_out, const float *residual, float *y,
                    float *y_norm, float eps) {
  double *row = (double *)malloc(sizeof(double) * (size_t)H);
  for (int t = 0; t < T; t++) {
    double ss = 0.0;
    for (int j = 0; j < H; j++) {
      double v = 0.0;
      if (residual) v += (double)residual[(size_t)t * H + j];
      if (shared_out) v += (double)shared_out[(size_t)t * H + j];
      for (int k = 0; k < K; k++)
        v += (double)w[(size_t)t * K + k] * (double)expert_out[((size_t)t * K + k) * H + j];
      row[j] = v;
      ss += v * v;
    }
    double inv = 1.0 / sqrt(ss / H + (double)eps);
    for (int j = 0; j < H; j++) {
      y[(size_t)t * H + j] = (float)row[j];
      if (y_norm) y_norm[(size_t)t * H + j] = (float)(row[j] * inv);
    }
  }
  free(row);
}

void oracle_rmsnorm(int T, int H, const float *x, float *y, float eps) {
  for (int t = 0; t < T; t++) {
    double ss = 0.0;
    for (int j = 0; j < H; j++) ss += (double)x[(size_t)t * H + j] * x[(size_t)t * H + j];
    double inv = 1.0 / sqrt(ss / H + (double)eps);
    for (int j = 0; j < H; j++) y[(size_t)t * H + j] = (float)(x[(size_t)t * H + j] * inv);
  }
}

/* Number of OpenMP threads the oracle's parallel loops use (1 without OpenMP). */
#ifdef _OPENMP
#include <omp.h>
int oracle_threads(void) { return omp_get_max_threads(); }
void oracle_set_threads(int n) { omp_set_num_threads(n > 0 ? n : 1); }
#else
int oracle_threads(void) { return 1; }
void oracle_set_threads(int n) { (void)n; }
#endif
