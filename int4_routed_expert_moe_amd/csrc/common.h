// Device helpers shared by the libmoe kernels (gfx950, wave64).
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

#define QBLK 32
#define WAVE 64

namespace moe {

// --- wave reductions (wave64) ----------------------------------------------
// DPP moves stay in the VALU (no LDS round trip per step, unlike the
// ds_bpermute that __shfl_xor lowers to).  Lanes a DPP move does not write
// receive `old` (0 here, the identity of the sum).
template <int CTRL, int ROW_MASK = 0xf, int BANK_MASK = 0xf>
__device__ __forceinline__ float dpp_f(float v) {
  return __int_as_float(
      __builtin_amdgcn_update_dpp(0, __float_as_int(v), CTRL, ROW_MASK, BANK_MASK, true));
}

// Sum over the 64 lanes, returned to every lane: pairs and quads by
// quad_perm, rows of 16 by two rotations, then rows 0+1 and 2+3 by the row
// broadcasts of lanes 15 and 31; lane 63 ends with the total.
__device__ __forceinline__ float wave_sum(float v) {
  v += dpp_f<0xB1>(v);        // quad_perm [1,0,3,2]
  v += dpp_f<0x4E>(v);        // quad_perm [2,3,0,1]
  v += dpp_f<0x124>(v);       // row_ror:4
  v += dpp_f<0x128>(v);       // row_ror:8
  v += dpp_f<0x142, 0xA>(v);  // row_bcast:15 -> rows 1 and 3
  v += dpp_f<0x143, 0xC>(v);  // row_bcast:31 -> rows 2 and 3
  return __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), 63));
}

__device__ __forceinline__ float wave_max(float v) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) v = fmaxf(v, __shfl_xor(v, o, WAVE));
  return v;
}

// --- the router's fixed-order sigmoid -------------------------------------
// e^y in fp32 from basic operations only, so that every kernel and a CPU
// following the same steps get the same bits: y clamped to [-87, 87];
// Cody–Waite reduction n = rint(y log2 e), r = (y - n LN2_HI) - n LN2_LO with
// ln 2 split into a 16-bit-exact high part and the fp32 remainder; the
// degree-7 Taylor polynomial of e^r (coefficients fp32(1/k!)) in Horner form
// with fma; then the scaling by 2^n.  Files using it are compiled with
// -ffp-contract=off and correctly rounded fp32 division.
__device__ __forceinline__ float exp_fixed(float y) {
  y = y > 87.0f ? 87.0f : y;
  y = y < -87.0f ? -87.0f : y;
  const float n = __builtin_rintf(y * 1.44269502f);
  float r = __builtin_fmaf(-n, 0.693145751953125f, y);
  r = __builtin_fmaf(-n, 1.42860677e-06f, r);
  float p = 1.98412701e-04f;                  // 1/7!
  p = __builtin_fmaf(p, r, 1.38888892e-03f);  // 1/6!
  p = __builtin_fmaf(p, r, 8.33333377e-03f);  // 1/5!
  p = __builtin_fmaf(p, r, 4.16666679e-02f);  // 1/4!
  p = __builtin_fmaf(p, r, 1.66666672e-01f);  // 1/3!
  p = __builtin_fmaf(p, r, 0.5f);
  p = __builtin_fmaf(p, r, 1.0f);
  p = __builtin_fmaf(p, r, 1.0f);
  return __builtin_ldexpf(p, (int)n);
}

// sigmoid(l) = 1 / (1 + e^-l), correctly rounded division.
__device__ __forceinline__ float sigmoid_fixed(float l) { return 1.0f / (1.0f + exp_fixed(-l)); }

// --- order-preserving key of a float (no NaN); -0 is folded onto +0 -------
__device__ __forceinline__ uint32_t float_key(float f) {
  f = f + 0.0f;
  uint32_t u = __float_as_uint(f);
  return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}

// --- packed int4 -> int8 lanes ---------------------------------------------
// A 32-bit word holds 8 codes: byte i = (code 2i in bits 0..3, code 2i+1 in
// bits 4..7).  lo16 returns the even codes times 16 as four int8, hi16 the
// odd codes times 16; the sign of each nibble lands on the int8 sign bit.
__device__ __forceinline__ int lo16(uint32_t v) { return (int)((v << 4) & 0xF0F0F0F0u); }
__device__ __forceinline__ int hi16(uint32_t v) { return (int)(v & 0xF0F0F0F0u); }

// Even / odd bytes of the 8 int8 activations (w0 = bytes 0..3, w1 = 4..7).
__device__ __forceinline__ int even_bytes(uint32_t w0, uint32_t w1) {
  return (int)__builtin_amdgcn_perm(w1, w0, 0x06040200u);
}
__device__ __forceinline__ int odd_bytes(uint32_t w0, uint32_t w1) {
  return (int)__builtin_amdgcn_perm(w1, w0, 0x07050301u);
}

__device__ __forceinline__ int sdot4(int a, int b, int c) {
  return __builtin_amdgcn_sdot4(a, b, c, false);
}

// Q8_0 activation block pre-split for the int4 dot: ev[j] = bytes
// (8j, 8j+2, 8j+4, 8j+6), od[j] = (8j+1, 8j+3, 8j+5, 8j+7), j = 0..3.
struct QBlock {
  int ev[4];
  int od[4];
};

__device__ __forceinline__ QBlock split_block(const uint4 a, const uint4 b) {
  QBlock r;
  r.ev[0] = even_bytes(a.x, a.y);
  r.od[0] = odd_bytes(a.x, a.y);
  r.ev[1] = even_bytes(a.z, a.w);
  r.od[1] = odd_bytes(a.z, a.w);
  r.ev[2] = even_bytes(b.x, b.y);
  r.od[2] = odd_bytes(b.x, b.y);
  r.ev[3] = even_bytes(b.z, b.w);
  r.od[3] = odd_bytes(b.z, b.w);
  return r;
}

// Exact dot of 32 int4 codes (16 bytes, w) with 32 int8 activations: returns
// 16 * sum(code * q).  |result| <= 16 * 32 * 8 * 127 < 2^20.
__device__ __forceinline__ int dot_int4_block16(const uint4 w, const QBlock &a) {
  int acc = 0;
  acc = sdot4(lo16(w.x), a.ev[0], acc);
  acc = sdot4(hi16(w.x), a.od[0], acc);
  acc = sdot4(lo16(w.y), a.ev[1], acc);
  acc = sdot4(hi16(w.y), a.od[1], acc);
  acc = sdot4(lo16(w.z), a.ev[2], acc);
  acc = sdot4(hi16(w.z), a.od[2], acc);
  acc = sdot4(lo16(w.w), a.ev[3], acc);
  acc = sdot4(hi16(w.w), a.od[3], acc);
  return acc;
}

// --- packed int2 -> int8 lanes ---------------------------------------------
// A byte holds 4 codes (code i in bits 2i..2i+1).  For a 32-bit word (16
// codes), field f in {0,1,2,3} of every byte shifted to bits 6..7 gives 64 *
// code as int8; q needs bytes (4j+f) of the block, gathered per field.
__device__ __forceinline__ int int2_field64(uint32_t v, int f) {
  return (int)((v << (6 - 2 * f)) & 0xC0C0C0C0u);
}

// Activations of one 64-element int2 piece split by field: a[f][j] holds
// bytes (16j + 4i + f), i = 0..3 ... see gather_int2.
struct QBlock2 {
  int f[4][4];  // [field][word j]: bytes q[16j + f], q[16j + 4 + f], q[16j+8+f], q[16j+12+f]
};

// Four int8 bytes selected from two words with byte selectors (v_perm).
__device__ __forceinline__ int perm2(uint32_t lo, uint32_t hi, uint32_t sel) {
  return (int)__builtin_amdgcn_perm(hi, lo, sel);
}

// A load through the global address space.  Record addresses read from
// memory (the caller's pointer table, the slot table) are generic to the
// compiler, which would otherwise emit flat loads for every weight piece.
#define MOE_GLOBAL __attribute__((address_space(1)))
template <class T>
__device__ __forceinline__ T gload(const uint8_t *base, size_t off) {
  const MOE_GLOBAL uint8_t *g = (const MOE_GLOBAL uint8_t *)base;
  return *(const MOE_GLOBAL T *)(g + off);
}
typedef unsigned int moe_u32x4 __attribute__((ext_vector_type(4)));
template <>
__device__ __forceinline__ uint4 gload<uint4>(const uint8_t *base, size_t off) {
  const MOE_GLOBAL uint8_t *g = (const MOE_GLOBAL uint8_t *)base;
  const moe_u32x4 v = *(const MOE_GLOBAL moe_u32x4 *)(g + off);
  return make_uint4(v.x, v.y, v.z, v.w);
}

// A 16-byte weight piece read once per step: a non-temporal load, which
// streams past the caches instead of filling them (measured on a plain
// streaming read: ~6.9 TB/s against ~6.2 TB/s with ordinary loads).
#ifndef MOE_NT_WEIGHTS
#define MOE_NT_WEIGHTS 1
#endif
__device__ __forceinline__ uint4 gload_stream(const uint8_t *base, size_t off) {
  const MOE_GLOBAL uint8_t *g = (const MOE_GLOBAL uint8_t *)base;
#if MOE_NT_WEIGHTS
  const moe_u32x4 v = __builtin_nontemporal_load((const MOE_GLOBAL moe_u32x4 *)(g + off));
#else
  const moe_u32x4 v = *(const MOE_GLOBAL moe_u32x4 *)(g + off);
#endif
  return make_uint4(v.x, v.y, v.z, v.w);
}

// Weight-format tags of the kernels: 8, 4, 2 = integer codes of that many
// bits with one fp32 scale per row; WB_MX = MXFP4 ("Comment exécuter un
// réseau de neurones de 744 milliards de paramètres…", section "Modèles
// supportés": native MXFP4 weights) -- FP4 E2M1 codes packed like int4, one
// E8M0 scale byte per 32 codes of a row, no row scale.
constexpr int WB_MX = 5;
// WB_F8 = FP8 E4M3 codes, one byte per element, one fp32 scale per 128x128
// block, no row scale ("Comment exécuter…", section "Modèles supportés":
// fp4/fp8 weights; "Show HN…", converter item: 128x128 block scales).
constexpr int WB_F8 = 9;
template <int WB>
__host__ __device__ constexpr int code_bits() {
  return WB == WB_MX ? 4 : WB == WB_F8 ? 8 : WB;
}
// Byte-wide codes: activation pieces of 16 codes (half a Q8_0 block).
__host__ __device__ constexpr bool byte_codes(int WB) { return WB == 8 || WB == WB_F8; }

typedef float f8v2 __attribute__((ext_vector_type(2)));

// Marks a weight piece as changed (an empty asm, registers only), so the
// compiler converts FP8 codes where they are used instead of hoisting every
// converted value out of a token loop (16 live registers per piece).
__device__ __forceinline__ void opaque_words(uint4 &v) {
  asm volatile("" : "+v"(v.x), "+v"(v.y), "+v"(v.z), "+v"(v.w));
}

// acc + sum over the 4 bytes of w (FP8 E4M3 codes) and of x (int8) of
// 512 fp8(c) q: gfx950's OCP E4M3 conversion scaled by 512 gives exact
// integers of at most 18 bits, multiplied in 24-bit integer multiply-adds
// (|512 fp8| <= 229376, so 16 such products stay below 2^31).
__device__ __forceinline__ int dot_fp8_word(uint32_t w, uint32_t x, int acc) {
  const f8v2 lo = __builtin_amdgcn_cvt_scalef32_pk_f32_fp8(w, 512.0f, false);
  const f8v2 hi = __builtin_amdgcn_cvt_scalef32_pk_f32_fp8(w, 512.0f, true);
  acc = __mul24((int)lo.x, (int)(int8_t)x) + acc;
  acc = __mul24((int)lo.y, (int)(int8_t)(x >> 8)) + acc;
  acc = __mul24((int)hi.x, (int)(int8_t)(x >> 16)) + acc;
  acc = __mul24((int)hi.y, (int)(int8_t)(x >> 24)) + acc;
  return acc;
}

// E8M0 scale byte -> 2^(s-127) as fp32 (s = 0 gives the subnormal 2^-127).
__device__ __forceinline__ float e8m0_float(uint32_t s) {
  return __uint_as_float(s ? s << 23 : 0x00400000u);
}

// FP4 E2M1 codes in the low (shift 0) or high (shift 4) nibbles of a word's
// four bytes -> four int8 lanes of twice their value (0, 1, 2, 3, 4, 6, 8,
// 12 with the code's sign): magnitudes by byte lookup (v_perm_b32 selectors
// 0-7), the negative table picked where the sign bit is set.  The per-byte
// mask comes from v_perm_b32's sign-replicating selectors 8-11 (the top bit
// of bytes 1, 3, 5, 7 of the 8-byte input): with the codes shifted so that
// each sign bit is the top bit of one of those bytes, one v_perm yields
// 0xFF or 0x00 per lane.
__device__ __forceinline__ int mx_lanes(uint32_t w, int shift) {
  const uint32_t sel = (w >> shift) & 0x07070707u;
  const uint32_t pos = __builtin_amdgcn_perm(0x0C080604u, 0x03020100u, sel);
  const uint32_t neg = __builtin_amdgcn_perm(0xF4F8FAFCu, 0xFDFEFF00u, sel);
  // the top bit of each byte of x is its code's sign bit (x = w << 4 for the
  // low nibbles, w for the high ones; the other bits do not matter): input
  // bytes 1, 3 = (x << 8) bytes 1, 3 hold the signs of code bytes 0, 2,
  // bytes 5, 7 = x bytes 1, 3 those of code bytes 1, 3
  const uint32_t x = w << (4 - shift);
  const uint32_t m = __builtin_amdgcn_perm(x, x << 8, 0x0B090A08u);
  return (int)((neg & m) | (pos & ~m));
}

// Exact dot of 32 FP4 codes (16 bytes) with 32 int8 activations split like
// the int4 ones: sum (2 fp4(c)) q, |result| <= 32 * 12 * 127.
__device__ __forceinline__ int dot_mx_block(const uint4 w, const QBlock &a) {
  int acc = 0;
  acc = sdot4(mx_lanes(w.x, 0), a.ev[0], acc);
  acc = sdot4(mx_lanes(w.x, 4), a.od[0], acc);
  acc = sdot4(mx_lanes(w.y, 0), a.ev[1], acc);
  acc = sdot4(mx_lanes(w.y, 4), a.od[1], acc);
  acc = sdot4(mx_lanes(w.z, 0), a.ev[2], acc);
  acc = sdot4(mx_lanes(w.z, 4), a.od[2], acc);
  acc = sdot4(mx_lanes(w.w, 0), a.ev[3], acc);
  acc = sdot4(mx_lanes(w.w, 4), a.od[3], acc);
  return acc;
}

// Record of routed expert e (0 <= e < E): entry e of the caller's table of
// record pointers when there is one (records may then sit anywhere the
// device can read: HBM cache slots, pinned host memory), else
// experts + e * blob_bytes.
template <class Args>
__device__ __forceinline__ const uint8_t *expert_record(const Args &a, int e) {
  return a.expert_ptrs ? a.expert_ptrs[e] : a.experts + (size_t)e * a.blob_bytes;
}

// Adaptive expert top-p ("Show HN…", section モデルのダウンロードと実行,
// options list) on one token's unbiased scores sv[0..K) in rank order, S
// their fp32 left-to-right sum: the number n of ranks kept, the first n with
// sv[0] + ... + sv[n-1] >= top_p * S (same order, fp32), and that sum in
// *S_kept.  top_p outside (0, 1) keeps every rank (S_kept = S).
__device__ __forceinline__ int top_p_keep(const float (&sv)[16], int K, float S, float top_p,
                                          float *S_kept) {
  *S_kept = S;
  if (!(top_p > 0.0f && top_p < 1.0f)) return K;
  const float thr = top_p * S;
  float c = 0.0f;
  int n = K;
#pragma unroll
  for (int k = 0; k < 16; k++) {
    if (k < K && n == K) {
      c = c + sv[k];
      if (c >= thr) {
        n = k + 1;
        *S_kept = c;
      }
    }
  }
  return n;
}

}  // namespace moe
