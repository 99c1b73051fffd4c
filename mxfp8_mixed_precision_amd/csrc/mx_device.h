// Device-side MXFP8 helpers for gfx950 (shared by the quantizer and the GEMM epilogues).
//
// The rule (OCP MX v1.0 MXFP8, with the formats named in afd-plugin PR #475 "quantize the
// A2E FFN transport to MXFP8", section "Purpose"): per 32-element group, scale byte
// = clamp(floor(log2 amax) - 8, -127, 127) + 127 and codes = E4M3 RNE(v / 2^(byte-127))
// saturated to +-448.
//
// Implementation on gfx950:
//  * amax is taken on BF16 bit patterns: with the sign cleared, the ordering of finite
//    BF16 magnitudes is the ordering of their 15-bit integers, so packed u16 max works.
//  * For a finite nonzero amax with exponent field ef, floor(log2 amax) - 8 + 127 = ef - 8
//    (ef >= 1); a subnormal or zero amax has ef = 0 and the clamp gives byte 0. So the
//    byte is max(ef - 8, 0), or 0xFF when ef = 255 (Inf/NaN present).
//  * Conversion uses v_cvt_scalef32_pk_fp8_bf16, which divides by the power-of-two scale
//    and rounds to nearest even with exact subnormals, but does not saturate (magnitudes
//    above 464 become NaN). Clamping |v| to 448 * 2^e first (exact in BF16: 1.75 *
//    2^(e+8)) makes it equal to round-then-saturate. The clamp is a packed u16 min on
//    the magnitude bits.
//  * The scale operand is 2^e as an fp32: bits byte << 23, and for byte 0 the fp32
//    subnormal 2^-127 (0x00400000) -- not the zero that byte << 23 would give.
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace mxf {

typedef unsigned short u16x2 __attribute__((ext_vector_type(2)));
typedef short s16x2 __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));

__device__ __forceinline__ uint32_t pk_max_u16(uint32_t a, uint32_t b) {
  return __builtin_bit_cast(uint32_t, __builtin_elementwise_max(__builtin_bit_cast(u16x2, a),
                                                                __builtin_bit_cast(u16x2, b)));
}
__device__ __forceinline__ uint32_t pk_min_u16(uint32_t a, uint32_t b) {
  return __builtin_bit_cast(uint32_t, __builtin_elementwise_min(__builtin_bit_cast(u16x2, a),
                                                                __builtin_bit_cast(u16x2, b)));
}

// Per-group scale state derived from the group's amax magnitude bits.
struct Scale {
  uint32_t lim2;     // clamp limit (magnitude bits of 448 * 2^e) in both u16 halves
  float xf;          // 2^e as fp32 (the cvt's scale operand)
  uint32_t nanmask;  // 0x7F7F7F7F for a non-finite group (forces NaN codes), else 0
  uint32_t byte;     // E8M0 byte
};

// Element formats: FMT_E4M3 (emax 8, largest 448 = 1.75 * 2^8) and FMT_E5M2 (emax 15, largest
// 57344 = 1.75 * 2^15). The rule is the same with the format's emax; the clamp limit is
// 1.75 * 2^(e + emax) and both formats' NaN code is 0x7F | sign.
enum { FMT_E4M3 = 0, FMT_E5M2 = 1 };

template <int FMT = FMT_E4M3>
__device__ __forceinline__ Scale scale_from_amax(uint32_t amax_bits) {
  constexpr uint32_t EMAX = FMT == FMT_E5M2 ? 15u : 8u;
  const uint32_t ef = amax_bits >> 7;
  Scale s;
  if (ef >= 255u) {
    s.byte = 255u;
    s.lim2 = 0u;
    s.xf = 1.0f;
    s.nanmask = 0x7F7F7F7Fu;
  } else {
    const uint32_t byte = ef > EMAX ? ef - EMAX : 0u;
    const uint32_t lim = ((byte + EMAX) << 7) | 0x60u;
    s.byte = byte;
    s.lim2 = lim | (lim << 16);
    s.xf = __uint_as_float(byte ? (byte << 23) : 0x00400000u);
    s.nanmask = 0u;
  }
  return s;
}

// Magnitude bits of two packed BF16 values.
__device__ __forceinline__ uint32_t mag2(uint32_t v) { return v & 0x7FFF7FFFu; }

// Two packed BF16 (lo, hi) -> two E4M3 codes written into the low (hi=false) or high
// (hi=true) 16 bits of `old`.
template <bool HI, int FMT = FMT_E4M3>
__device__ __forceinline__ uint32_t cvt2(uint32_t old, uint32_t v, const Scale& s) {
  const uint32_t c = (v & 0x80008000u) | pk_min_u16(v & 0x7FFF7FFFu, s.lim2);
  s16x2 r;
  if constexpr (FMT == FMT_E5M2)
    r = __builtin_amdgcn_cvt_scalef32_pk_bf8_bf16(__builtin_bit_cast(s16x2, old), __builtin_bit_cast(bf16x2, c),
                                                  s.xf, HI);
  else
    r = __builtin_amdgcn_cvt_scalef32_pk_fp8_bf16(__builtin_bit_cast(s16x2, old), __builtin_bit_cast(bf16x2, c),
                                                  s.xf, HI);
  return __builtin_bit_cast(uint32_t, r);
}

// Four BF16 (two packed words) -> four codes in one word (byte i = element i).
template <int FMT = FMT_E4M3>
__device__ __forceinline__ uint32_t cvt4(uint32_t v01, uint32_t v23, const Scale& s) {
  uint32_t r = cvt2<false, FMT>(0u, v01, s);
  r = cvt2<true, FMT>(r, v23, s);
  return r | s.nanmask;
}

// 16-byte store that bypasses the caches' retention (non-temporal): for outputs no kernel of
// the library reads back soon (the GEMM results, the tensors saved for the backward pass), so
// they do not evict operand panels that the running GEMMs re-read from L2.
__device__ __forceinline__ void store16_nt(void* dst, uint4 v) {
  typedef unsigned u32x4 __attribute__((ext_vector_type(4)));
  __builtin_nontemporal_store((u32x4){v.x, v.y, v.z, v.w}, reinterpret_cast<u32x4*>(dst));
}

__device__ __forceinline__ uint4 load16_nt(const void* src) {
  typedef unsigned u32x4 __attribute__((ext_vector_type(4)));
  const u32x4 v = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(src));
  return make_uint4(v.x, v.y, v.z, v.w);
}

// Value held by lane l ^ 1 (DPP quad permute [1,0,3,2]) and by lane l ^ 2 ([2,3,0,1]).
__device__ __forceinline__ uint32_t dpp_xor1(uint32_t v) {
  return (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0xB1, 0xF, 0xF, false);
}
__device__ __forceinline__ uint32_t dpp_xor2(uint32_t v) {
  return (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0x4E, 0xF, 0xF, false);
}

// Amax magnitude bits of 16 BF16 values held in 8 packed words.
__device__ __forceinline__ uint32_t amax16(const uint32_t* v) {
  uint32_t m = mag2(v[0]);
#pragma unroll
  for (int i = 1; i < 8; ++i) m = pk_max_u16(m, mag2(v[i]));
  return max(m & 0xFFFFu, m >> 16);
}

// Pack the low (or high) BF16 halves of two words: (a.lo, b.lo) or (a.hi, b.hi).
__device__ __forceinline__ uint32_t pack_lo(uint32_t a, uint32_t b) {
  return __builtin_amdgcn_perm(b, a, 0x05040100u);
}
__device__ __forceinline__ uint32_t pack_hi(uint32_t a, uint32_t b) {
  return __builtin_amdgcn_perm(b, a, 0x07060302u);
}

// fp32 -> BF16 bits, round to nearest even (gfx950 hardware conversion).
__device__ __forceinline__ uint32_t bf16_bits(float f) {
  return (uint32_t)__builtin_bit_cast(unsigned short, (__bf16)f);
}
// Two fp32 values -> a packed BF16 pair (lo in bits 0-15), each rounded to nearest even: one
// gfx950 two-lane conversion instead of two conversions and a pack.
typedef float f32x2 __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
__device__ __forceinline__ uint32_t bf16x2_bits(float lo, float hi) {
  return __builtin_bit_cast(uint32_t, __builtin_convertvector((f32x2){lo, hi}, bf16x2));
}
// The two halves of a packed BF16 pair as fp32 (exact).
__device__ __forceinline__ float bf16_lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t w) { return __uint_as_float(w & 0xFFFF0000u); }

// sigmoid(g) = 1 / (1 + 2^(-g log2 e)) from the hardware base-2 exponential and reciprocal
// (each within about 1 ulp); every caller rounds its result to BF16. No select on the sign:
// for g below about -87 the exponential reaches +inf (or the reciprocal leaves the fp32
// normal range) and the result is 0 or a flushed denormal, where sigmoid itself is below
// 2^-126; it is never NaN for a finite g.
__device__ __forceinline__ float sigmoid_f(float g) {
  return __builtin_amdgcn_rcpf(1.0f + __builtin_amdgcn_exp2f(-g * 1.44269504088896340736f));
}

// The SwiGLU rounding points (shared by the fused GEMM epilogues and the standalone kernels, so
// both compute bit-identical values): from the BF16 g, u of the FC1 output,
// h = BF16(silu(g) * u); in backward, from BF16 dh, dG = BF16(dh u s (1 + g (1 - s))) and
// dU = BF16(dh g s) with s = sigmoid(g). Arguments and results are BF16 bit patterns.
// The helpers take and return packed BF16 pairs (two elements per 32-bit word).
__device__ __forceinline__ float silu_mul(float gf, float uf) { return gf * sigmoid_f(gf) * uf; }
__device__ __forceinline__ uint32_t swiglu_h2(uint32_t g2, uint32_t u2) {
  return bf16x2_bits(silu_mul(bf16_lo(g2), bf16_lo(u2)), silu_mul(bf16_hi(g2), bf16_hi(u2)));
}
__device__ __forceinline__ void dswiglu_f(float dh, float gf, float uf, float& dg, float& du) {
  const float sg = sigmoid_f(gf);
  dg = dh * uf * sg * (1.0f + gf * (1.0f - sg));
  du = dh * gf * sg;
}
__device__ __forceinline__ void dswiglu2(uint32_t dh2, uint32_t g2, uint32_t u2, uint32_t& dg2, uint32_t& du2) {
  float dg0, du0, dg1, du1;
  dswiglu_f(bf16_lo(dh2), bf16_lo(g2), bf16_lo(u2), dg0, du0);
  dswiglu_f(bf16_hi(dh2), bf16_hi(g2), bf16_hi(u2), dg1, du1);
  dg2 = bf16x2_bits(dg0, dg1);
  du2 = bf16x2_bits(du0, du1);
}

// Device-side check of the token-offset contract, done by one whole wavefront; every lane
// returns the same answer. offs [E+1], counts [E] or null.
__device__ __forceinline__ bool offsets_valid(const int32_t* offs, const int32_t* counts, int E,
                                              int pad, int64_t mcap) {
  const int lane = threadIdx.x & 63;
  bool bad = false;
  for (int i = lane; i <= E; i += 64) {
    const int32_t o = offs[i];
    if (o % pad != 0 || o < 0 || (int64_t)o > mcap) bad = true;
    if (i == 0 && o != 0) bad = true;
    if (i > 0) {
      const int32_t p = offs[i - 1];
      if (o < p) bad = true;
      if (counts) {
        const int32_t c = counts[i - 1];
        if (c < 0 || c > o - p) bad = true;
      }
    }
  }
  return !__any(bad);
}

// The token offsets read once by a whole wavefront (E < 64: lane i holds offs[i] and
// counts[i-1]): validity as in offsets_valid, offs[E], and -- with expert() -- the expert that
// owns a row, from a ballot instead of a chain of dependent loads. Every lane sees the same
// answers. For E >= 64 the members fall back to the looping helpers.
struct Offsets {
  const int32_t* offs;
  const int32_t* counts;
  int E;
  int32_t o;     // offs[lane] (lanes 0..E)
  int32_t c;     // real rows of expert lane - 1 (lanes 1..E)
  bool ok;
  int64_t mend;  // offs[E]
  __device__ __forceinline__ int expert(int64_t m) const;
  // end of expert e's real rows, offs[e] + counts[e] (e wavefront-uniform)
  __device__ __forceinline__ int64_t real_end(int e) const;
};

__device__ __forceinline__ bool offsets_valid(const int32_t* offs, const int32_t* counts, int E,
                                              int pad, int64_t mcap);

// Expert that owns row m (offs[e] <= m < offs[e+1]); requires m < offs[E].
__device__ __forceinline__ int expert_of_row(const int32_t* offs, int E, int64_t m) {
  int lo = 0, hi = E;  // invariant: offs[lo] <= m < offs[hi]
  while (hi - lo > 1) {
    const int mid = (lo + hi) >> 1;
    if ((int64_t)offs[mid] <= m) lo = mid; else hi = mid;
  }
  return lo;
}

}  // namespace mxf

namespace mxf {

__device__ __forceinline__ Offsets read_offsets(const int32_t* offs, const int32_t* counts, int E, int pad,
                                                int64_t mcap) {
  Offsets r;
  r.offs = offs;
  r.counts = counts;
  r.E = E;
  r.o = 0;
  r.c = 0;
  if (E >= 64) {
    r.ok = offsets_valid(offs, counts, E, pad, mcap);
    r.mend = r.ok ? offs[E] : 0;
    return r;
  }
  const int lane = threadIdx.x & 63;
  const bool in = lane <= E;
  const int32_t o = in ? offs[lane] : 0;
  const int32_t c = (counts && lane >= 1 && in) ? counts[lane - 1] : 0;
  const int32_t prev = __shfl_up(o, 1);
  bool bad = false;
  if (in) {
    if (o % pad != 0 || o < 0 || (int64_t)o > mcap) bad = true;
    if (lane == 0 && o != 0) bad = true;
    if (lane > 0) {
      if (o < prev) bad = true;
      if (counts && (c < 0 || c > o - prev)) bad = true;
    }
  }
  r.o = o;
  r.c = counts ? c : o - prev;
  r.ok = !__any(bad);
  r.mend = __builtin_amdgcn_readlane(o, E);  // uniform (SGPR) copy
  return r;
}

__device__ __forceinline__ int64_t Offsets::real_end(int e) const {
  if (E >= 64) return (int64_t)offs[e] + (counts ? counts[e] : offs[e + 1] - offs[e]);
  return (int64_t)__builtin_amdgcn_readlane(o, e) + __builtin_amdgcn_readlane(c, e + 1);
}

__device__ __forceinline__ int Offsets::expert(int64_t m) const {
  if (E >= 64) return expert_of_row(offs, E, m);
  const int lane = threadIdx.x & 63;
  // e = #{i in [1, E-1] : offs[i] <= m} (offs is non-decreasing and offs[0] = 0 <= m)
  return __popcll(__ballot(lane >= 1 && lane < E && (int64_t)o <= m));
}

}  // namespace mxf
