/*
 * Seeded synthetic inputs for one routed-MoE layer (host side).
 *
 * What lives here: counter-based random draws, an approximately normal
 * variate built from them, uniform variates, and the offline step that turns
 * float expert weights into packed low-bit codes with one fp32 scale per row
 * (the pages' engine gets its expert container from an offline converter;
 * "colibrì … Show HN" page, implemented-features list, converter item).
 * What does not live here: any arithmetic of the layer itself (router,
 * Q8_0, integer dots, SwiGLU, combine).  Both the CPU oracle and the HIP
 * library consume the bytes written here; a GPU copy of the same generator
 * (synth_gpu.hip) writes identical bytes for the large weight sets.
 *
 * Generator definitions (all exact integer or correctly rounded fp32 steps,
 * so a GPU implementation reproduces them bit for bit):
 *   mix64        SplitMix64 output function (Steele, Lea, Flood, OOPSLA 2014)
 *   draw(key,i)  = mix64(key + (i+1)*0x9E3779B97F4A7C15)   (i-th stream value)
 *   normal(key,i) = (S - 393210) / 65536, S = sum of the twelve 16-bit fields of
 *                  draw(key,3i), draw(key,3i+1), draw(key,3i+2)
 *                  (Irwin–Hall sum of 12 uniforms: mean 0, variance ~1, |z| <= 6)
 *   uniform(key,i) = (draw(key,i) >> 40) * 2^-24  in [0,1)
 *
 * Packed weight record of one expert (wbits = 8, 4 or 2), rows of the three
 * matrices followed by their fp32 per-row scales:
 *   gate codes [I][H*wbits/8] | up codes [I][H*wbits/8] | down codes [H][I*wbits/8]
 *   | gate scale [I] | up scale [I] | down scale [H]
 * int4: element 2j in the low nibble of byte j, 2j+1 in the high nibble,
 *       two's complement; int2: element 4j+i in bits 2i..2i+1, two's complement;
 *       int8: one two's-complement byte per element.
 * Row quantiser: amax = max|w|, s = amax / qdiv (qdiv 127 for int8, 7 for
 *   int4, 2 for int2), code = clamp(roundf(w / s), qlo, qhi) (int8: [-127,127],
 *   int4: [-8,7], int2: [-2,1]); s = 0 -> codes 0.
 *
 * MXFP4 record (wbits code -4; the OCP microscaling format that one of the
 * pages' supported models ships its weights in): FP4 E2M1 codes two per byte
 * (element 2j in the low nibble) for the three matrices in the same order,
 * then one E8M0 scale byte per 32 consecutive elements of a row: gate
 * [I][H/32], up [I][H/32], down [H][I/32].  Block quantiser: amax = max|w|
 * over the block, X = floor(log2 amax) - 2 (frexpf, exact; the largest FP4
 * magnitude is 6 = 1.5 * 2^2), scale byte X + 127 clamped to [1, 254]
 * (127 when amax = 0); each element v = w * 2^-X (exact) goes to the nearest
 * FP4 magnitude {0, .5, 1, 1.5, 2, 3, 4, 6}, ties to the even mantissa,
 * saturating at 6, sign in bit 3 (zero magnitude -> code 0).
 *
 * FP8 record (wbits code -8; the fp8 weights one of the pages' supported
 * models ships, with the 128x128 block scales its converter reads): one
 * OCP E4M3 byte per element for the three matrices in the same order, then
 * fp32 scales per 128x128 block: gate [I/128][H/128], up [I/128][H/128],
 * down [H/128][I/128].  Block quantiser: amax = max|w| over the block,
 * s = amax / 448 (s = 0 -> codes 0); each v = w / s (correctly rounded) goes
 * to the nearest E4M3 value, ties to the even mantissa, saturating at 448;
 * a zero magnitude is code 0.
 *
 * Build: gcc -O2 -fopenmp -ffp-contract=off -fno-fast-math -shared -fPIC
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

#define SYN_GOLDEN 0x9E3779B97F4A7C15ULL

static inline uint64_t mix64(uint64_t z) {
  z = (z ^ (z >> 30)) * 0xBF58476D1CE4E5B9ULL;
  z = (z ^ (z >> 27)) * 0x94D049BB133111EBULL;
  return z ^ (z >> 31);
}

static inline uint64_t draw(uint64_t key, uint64_t i) {
  return mix64(key + (i + 1) * SYN_GOLDEN);
}

static inline int32_t sum16(uint64_t v) {
  return (int32_t)(v & 0xFFFF) + (int32_t)((v >> 16) & 0xFFFF) +
         (int32_t)((v >> 32) & 0xFFFF) + (int32_t)(v >> 48);
}

static inline float normal_at(uint64_t key, uint64_t i) {
  int32_t s = sum16(draw(key, 3 * i)) + sum16(draw(key, 3 * i + 1)) +
              sum16(draw(key, 3 * i + 2));
  return (float)(s - 393210) * (1.0f / 65536.0f);
}

uint64_t synth_draw(uint64_t key, uint64_t i) { return draw(key, i); }

uint64_t synth_key(uint64_t seed, uint32_t layer, uint32_t tensor,
                   uint32_t expert, uint32_t matrix) {
  uint64_t k = mix64(seed + SYN_GOLDEN);
  k = mix64(k ^ (((uint64_t)layer << 32) | tensor));
  k = mix64(k ^ (((uint64_t)expert << 32) | matrix));
  return k;
}

/* out[i] = sigma * normal(key, start + i) */
void synth_normal_fill(uint64_t key, uint64_t start, int64_t n, float sigma,
                       float *out) {
#pragma omp parallel for schedule(static) if (n > 65536)
  for (int64_t i = 0; i < n; i++) out[i] = normal_at(key, start + (uint64_t)i) * sigma;
}

/* out[i] = lo + (hi - lo) * uniform(key, start + i) */
void synth_uniform_fill(uint64_t key, uint64_t start, int64_t n, float lo,
                        float hi, float *out) {
  for (int64_t i = 0; i < n; i++) {
    float u = (float)(draw(key, start + (uint64_t)i) >> 40) * 0x1p-24f;
    out[i] = lo + (hi - lo) * u;
  }
}

#define SYN_MXFP4 (-4)
#define SYN_FP8 (-8)

size_t synth_blob_bytes(int H, int I, int wbits) {
  const size_t elems = (size_t)2 * I * H + (size_t)H * I;
  if (wbits == SYN_MXFP4) return elems / 2 + elems / 32;
  if (wbits == SYN_FP8) return elems + sizeof(float) * 3 * (size_t)(I / 128) * (H / 128);
  return elems * (size_t)wbits / 8 + sizeof(float) * ((size_t)2 * I + H);
}

/* FP4 E2M1 code of w at block exponent X (see the header). */
static unsigned fp4_code(float w, int X) {
  const float v = fabsf(ldexpf(w, -X));
  unsigned m;
  if (v <= 0.25f) m = 0;
  else if (v < 0.75f) m = 1;
  else if (v <= 1.25f) m = 2;
  else if (v < 1.75f) m = 3;
  else if (v <= 2.5f) m = 4;
  else if (v < 3.5f) m = 5;
  else if (v <= 5.0f) m = 6;
  else m = 7;
  return m == 0 ? 0u : (m | (w < 0.0f ? 8u : 0u));
}

/* E4M3 code of v = w / s (see the header): exact steps only (frexpf,
 * ldexpf, rintf in round-to-nearest-even). */
static unsigned fp8_code(float v) {
  const unsigned sign = v < 0.0f ? 0x80u : 0u;
  const float a = fabsf(v);
  unsigned code;
  if (a >= 448.0f) {
    code = 0x7E;
  } else {
    int ex;
    frexpf(a, &ex); /* a = f 2^ex, f in [0.5, 1): floor(log2 a) = ex - 1 */
    const int E = ex - 1;
    if (a == 0.0f) {
      code = 0;
    } else if (E < -6) { /* subnormal: units of 2^-9; 8 units = 2^-6 = code 0x08 */
      code = (unsigned)rintf(ldexpf(a, 9));
    } else {
      int q = (int)rintf(ldexpf(a, 3 - E)); /* in [8, 16] */
      int EE = E;
      if (q == 16) {
        q = 8;
        EE++;
      }
      code = ((unsigned)(EE + 7) << 3) | (unsigned)(q - 8);
      if (code > 0x7E) code = 0x7E;
    }
  }
  return code == 0 ? 0u : (sign | code);
}

/* FP8 record for (seed, layer, expert): each 128x128 block of a matrix is
 * drawn twice (its amax first, then its codes), so no block is held. */
static int fp8_expert_blob(uint64_t seed, uint32_t layer, uint32_t expert, int H, int I,
                           float sigma, uint8_t *blob) {
  if (H <= 0 || I <= 0 || H % 128 || I % 128) return -1;
  const size_t gate_b = (size_t)I * H;
  uint8_t *codes[3] = {blob, blob + gate_b, blob + 2 * gate_b};
  float *sc = (float *)(blob + 3 * gate_b);
  const size_t nb = (size_t)(I / 128) * (H / 128);
  float *scl[3] = {sc, sc + nb, sc + 2 * nb};
  const int rows[3] = {I, I, H}, cols[3] = {H, H, I};
  for (int m = 0; m < 3; m++) {
    const uint64_t key = synth_key(seed, layer, 4u + (uint32_t)m, expert, (uint32_t)m);
    const int n = cols[m], rb = rows[m] / 128, cb = n / 128;
#pragma omp parallel for schedule(static)
    for (int blk = 0; blk < rb * cb; blk++) {
      const int br = blk / cb, bc = blk % cb;
      float amax = 0.0f;
      for (int r = br * 128; r < br * 128 + 128; r++)
        for (int c = bc * 128; c < bc * 128 + 128; c++)
          amax = fmaxf(amax, fabsf(normal_at(key, (uint64_t)r * (uint64_t)n + (uint64_t)c) * sigma));
      const float s = amax / 448.0f;
      scl[m][blk] = s;
      for (int r = br * 128; r < br * 128 + 128; r++)
        for (int c = bc * 128; c < bc * 128 + 128; c++) {
          const float w = normal_at(key, (uint64_t)r * (uint64_t)n + (uint64_t)c) * sigma;
          codes[m][(size_t)r * n + c] = (uint8_t)(s != 0.0f ? fp8_code(w / s) : 0u);
        }
    }
  }
  return 0;
}

/* One MXFP4 block: 32 floats -> 16 code bytes and the E8M0 scale byte. */
static void mx_block(const float *w, uint8_t *codes, uint8_t *scale) {
  float amax = 0.0f;
  for (int k = 0; k < 32; k++) amax = fmaxf(amax, fabsf(w[k]));
  int s = 127;
  if (amax > 0.0f) {
    int ex;
    frexpf(amax, &ex);  /* amax = f * 2^ex, f in [0.5, 1): floor(log2 amax) = ex - 1 */
    s = ex - 1 - 2 + 127;
    s = s < 1 ? 1 : (s > 254 ? 254 : s);
  }
  *scale = (uint8_t)s;
  for (int j = 0; j < 16; j++)
    codes[j] = (uint8_t)(fp4_code(w[2 * j], s - 127) | (fp4_code(w[2 * j + 1], s - 127) << 4));
}

/* One weight row: n float draws (sigma * normal), quantised and packed. */
static void quant_row(uint64_t key, uint64_t row, int n, int wbits, float sigma,
                      uint8_t *dst, float *scale, float *wbuf) {
  float amax = 0.0f;
  for (int c = 0; c < n; c++) {
    float w = normal_at(key, row * (uint64_t)n + (uint64_t)c) * sigma;
    wbuf[c] = w;
    amax = fmaxf(amax, fabsf(w));
  }
  const float qdiv = (wbits == 8) ? 127.0f : (wbits == 4) ? 7.0f : 2.0f;
  const int qlo = (wbits == 8) ? -127 : (wbits == 4) ? -8 : -2;
  const int qhi = (wbits == 8) ? 127 : (wbits == 4) ? 7 : 1;
  float s = amax / qdiv;
  *scale = s;
  const int per = 8 / wbits;
  const unsigned mask = (1u << wbits) - 1u;
  for (int j = 0; j < n / per; j++) {
    unsigned byte = 0;
    for (int i = 0; i < per; i++) {
      int q = 0;
      if (s != 0.0f) {
        float r = roundf(wbuf[j * per + i] / s);
        q = (int)r;
        if (q < qlo) q = qlo;
        if (q > qhi) q = qhi;
      }
      byte |= ((unsigned)q & mask) << (wbits * i);
    }
    dst[j] = (uint8_t)byte;
  }
}

/* Float weights of one matrix row before quantisation (for tests of the record). */
void synth_weight_row(uint64_t seed, uint32_t layer, uint32_t expert,
                      uint32_t matrix, int n, int row, float sigma, float *out) {
  uint64_t key = synth_key(seed, layer, 4u + matrix, expert, matrix);
  for (int c = 0; c < n; c++)
    out[c] = normal_at(key, (uint64_t)row * (uint64_t)n + (uint64_t)c) * sigma;
}

/* Expert record for (seed, layer, expert); matrix m = 0 gate, 1 up, 2 down. */
static int mx_expert_blob(uint64_t seed, uint32_t layer, uint32_t expert, int H, int I,
                          float sigma, uint8_t *blob) {
  if (H <= 0 || I <= 0 || H % 32 || I % 32) return -1;
  const size_t gate_b = (size_t)I * H / 2, down_b = (size_t)H * I / 2;
  uint8_t *codes[3] = {blob, blob + gate_b, blob + 2 * gate_b};
  uint8_t *sb = blob + 2 * gate_b + down_b;
  uint8_t *scl[3] = {sb, sb + (size_t)I * (H / 32), sb + 2 * (size_t)I * (H / 32)};
  const int rows[3] = {I, I, H}, cols[3] = {H, H, I};
  for (int m = 0; m < 3; m++) {
    const uint64_t key = synth_key(seed, layer, 4u + (uint32_t)m, expert, (uint32_t)m);
    const int n = cols[m];
#pragma omp parallel
    {
      float *wbuf = (float *)malloc(sizeof(float) * (size_t)n);
#pragma omp for schedule(static)
      for (int r = 0; r < rows[m]; r++) {
        for (int c = 0; c < n; c++)
          wbuf[c] = normal_at(key, (uint64_t)r * (uint64_t)n + (uint64_t)c) * sigma;
        for (int b = 0; b < n / 32; b++)
          mx_block(wbuf + 32 * b, codes[m] + (size_t)r * (n / 2) + 16 * b,
                   scl[m] + (size_t)r * (n / 32) + b);
      }
      free(wbuf);
    }
  }
  return 0;
}

int synth_expert_blob(uint64_t seed, uint32_t layer, uint32_t expert, int H,
                      int I, int wbits, float sigma, uint8_t *blob) {
  if (wbits == SYN_MXFP4) return mx_expert_blob(seed, layer, expert, H, I, sigma, blob);
  if (wbits == SYN_FP8) return fp8_expert_blob(seed, layer, expert, H, I, sigma, blob);
  if ((wbits != 8 && wbits != 4 && wbits != 2) || H <= 0 || I <= 0 || H % 8 || I % 8) return -1;
  const size_t gate_b = (size_t)I * H * wbits / 8;
  const size_t down_b = (size_t)H * I * wbits / 8;
  uint8_t *codes[3] = {blob, blob + gate_b, blob + 2 * gate_b};
  float *scales = (float *)(blob + 2 * gate_b + down_b);
  float *sc[3] = {scales, scales + I, scales + 2 * I};
  const int rows[3] = {I, I, H}, cols[3] = {H, H, I};
  for (int m = 0; m < 3; m++) {
    const uint64_t key = synth_key(seed, layer, 4u + (uint32_t)m, expert, (uint32_t)m);
    const int n = cols[m];
    const size_t row_b = (size_t)n * wbits / 8;
#pragma omp parallel
    {
      float *wbuf = (float *)malloc(sizeof(float) * (size_t)n);
#pragma omp for schedule(static)
      for (int r = 0; r < rows[m]; r++)
        quant_row(key, (uint64_t)r, n, wbits, sigma, codes[m] + (size_t)r * row_b,
                  sc[m] + r, wbuf);
      free(wbuf);
    }
  }
  return 0;
}
