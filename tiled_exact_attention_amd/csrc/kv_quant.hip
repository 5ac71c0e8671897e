// Appending new tokens to the int8 or int4 KV cache (the step before decode).
//
// Each (batch, token, kv head) row x of d values becomes d codes and one fp32
// scale: scale = absmax(x) / Q, code = clamp(rint(x / scale), -Q, Q) with
// ties to even, an all-zero row giving scale 0 and zero codes, Q = 127 for
// int8 codes and 7 for int4 codes (packed two per byte, element 2i in the low
// nibble of byte i).  This is the per-token, per-head symmetric scheme of the
// quantised cache; [FA-3MOVES] move 3 names the cache, not a scheme.  The codes decide integers, so every
// quotient x / scale is the correctly rounded IEEE fp32 one.
//
// Division: one correctly rounded reciprocal y = 1/scale per row, then per
// element q0 = x*y, r = fma(-q0, scale, x) (exact) and q = fma(r, y, q0),
// which is the correctly rounded quotient by Markstein's theorem (IBM J. Res.
// Dev. 34(1), 1990: y within half an ulp of 1/b, q0 within one ulp of a/b)
// as long as r stays a normal number for every quotient that can round to a
// non-zero code.  That holds for 2^-100 <= scale <= 2^120, which covers every
// finite row with absmax >= 2^-93; other rows take plain IEEE divisions.
//
// gfx950: the kernel is HBM-bound (2 or 4 bytes read and 1 written per
// element, half a byte for int4).  A row is handled by d/8 consecutive lanes,
// 8 values each; every lane group takes kRows rows spaced one block-pass apart
// and issues all their loads before any arithmetic, so each lane keeps 4-8
// 16-byte loads in flight.  The row's absmax is reduced with cross-lane xor
// shuffles; each lane stores its 8 codes as one 8-byte (int8) or 4-byte
// (int4) write into the head-major cache, the row's first lane the scale.
// The input rows and the codes carry the non-temporal hint (each byte is
// touched once); measured on MI355X for B32 T32768 Hkv8 d128 bf16 rows:
// int8 625 -> 604 us, int4 523 -> 510 us (the hint on the loads alone was
// slower, on the stores alone equal).
#include <type_traits>

#include "device_util.h"
#include "launch.h"

namespace fattn {
namespace {

constexpr int kThreads = 256;
constexpr int kRows = 4;  // rows per lane group

// I: row-index type, 32-bit whenever B*T*Hkv fits (the 64-bit divisions that
// map a row to its cache slot are emulated and cost ~10x more)
template <int D, typename T, typename I, int BITS>
__global__ __launch_bounds__(kThreads) void kv_quant_kernel(const T* __restrict__ x,
                                                            uint8_t* __restrict__ codes,
                                                            float* __restrict__ scales,
                                                            int64_t rows, int Tn, int Hkv,
                                                            int pos, int cap) {
  constexpr int L = D / 8;              // lanes per row
  constexpr float kQ = BITS == 8 ? 127.0f : 7.0f;
  constexpr int RB = D * BITS / 8;      // code bytes per row
  constexpr int RPP = kThreads / L;     // rows per block pass
  const int lane_in_row = threadIdx.x % L;
  const int64_t r0 = int64_t(blockIdx.x) * (RPP * kRows) + threadIdx.x / L;

  // raw bits first: all loads in flight before any arithmetic
  using Raw = typename std::conditional<sizeof(T) == 2, bf16x8, f32x4>::type;
  constexpr int kLoads = sizeof(T) == 2 ? 1 : 2;
  Raw raw[kRows][kLoads];
#pragma unroll
  for (int i = 0; i < kRows; ++i) {
    const int64_t r = r0 + int64_t(i) * RPP;
    const T* src = x + (r < rows ? r : 0) * D + 8 * lane_in_row;
#pragma unroll
    for (int j = 0; j < kLoads; ++j) raw[i][j] = __builtin_bit_cast(Raw, load_nt16(reinterpret_cast<const Raw*>(src) + j));
  }

#pragma unroll
  for (int i = 0; i < kRows; ++i) {
    const int64_t r = r0 + int64_t(i) * RPP;
    float v[8];
    if constexpr (sizeof(T) == 2) {
#pragma unroll
      for (int e = 0; e < 8; ++e) v[e] = float(raw[i][0][e]);
    } else {
#pragma unroll
      for (int e = 0; e < 4; ++e) { v[e] = raw[i][0][e]; v[4 + e] = raw[i][1][e]; }
    }
    float amax = 0.f;
#pragma unroll
    for (int e = 0; e < 8; ++e) amax = fmaxf(amax, fabsf(v[e]));
#pragma unroll
    for (int m = 1; m < L; m <<= 1) amax = fmaxf(amax, __shfl_xor(amax, m));
    const float scale = amax / kQ;
    const float y = 1.0f / scale;
    const bool exact_fma = scale >= 0x1p-100f && scale <= 0x1p120f;

    float q[8];
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      const float q0 = v[e] * y;
      q[e] = __builtin_fmaf(__builtin_fmaf(-q0, scale, v[e]), y, q0);
    }
    if (__builtin_expect(!exact_fma, 0)) {
#pragma unroll
      for (int e = 0; e < 8; ++e) q[e] = scale != 0.f ? v[e] / scale : 0.f;
    }
    // clamp, then round half to even by adding 1.5 * 2^23: the sum's ulp is 1,
    // so its low mantissa bits are the code in two's complement
    uint32_t lo = 0, hi = 0;
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      const float c = __builtin_amdgcn_fmed3f(q[e], -kQ, kQ) + 12582912.0f;
      if constexpr (BITS == 8) {
        const uint32_t byte = __float_as_uint(c) & 0xffu;
        if (e < 4) lo |= byte << (8 * e); else hi |= byte << (8 * (e - 4));
      } else {  // element e of the lane's 8 sits at bits 4e .. 4e+3 of one dword
        lo |= (__float_as_uint(c) & 0xfu) << (4 * e);
      }
    }
    if (r < rows) {
      const I ri = I(r);
      const I bt = ri / I(Hkv);
      const I h = ri - bt * I(Hkv);
      const I b = bt / I(Tn);
      const I t = bt - b * I(Tn);
      const int64_t slot = (int64_t(b) * Hkv + int64_t(h)) * int64_t(cap) + pos + int64_t(t);
      if constexpr (BITS == 8) {
        store_nt8(codes + slot * RB + 8 * lane_in_row, lo, hi);
      } else {
        store_nt4(codes + slot * RB + 4 * lane_in_row, lo);
      }
      if (lane_in_row == 0) scales[slot] = scale;
    }
  }
}

template <int D, typename T, typename I, int BITS>
hipError_t launch_idx(const KvQuantArgs& a, int64_t rows, hipStream_t stream) {
  constexpr int RPB = kThreads / (D / 8) * kRows;
  const int64_t blocks = (rows + RPB - 1) / RPB;
  if (blocks > 0x7fffffff) return hipErrorInvalidConfiguration;
  return launch_kernel(kv_quant_kernel<D, T, I, BITS>, dim3(unsigned(blocks)), dim3(kThreads), 0,
                       stream, static_cast<const T*>(a.x), static_cast<uint8_t*>(a.codes), a.scales,
                       rows, a.T, a.Hkv, a.pos, a.cap);
}

template <int D, typename T, int BITS>
hipError_t launch_bits(const KvQuantArgs& a, hipStream_t stream) {
  const int64_t rows = int64_t(a.B) * a.T * a.Hkv;
  if (rows <= 0xffffffffll) return launch_idx<D, T, uint32_t, BITS>(a, rows, stream);
  return launch_idx<D, T, uint64_t, BITS>(a, rows, stream);
}

template <int D, typename T>
hipError_t launch(const KvQuantArgs& a, hipStream_t stream) {
  if (a.bits == 8) return launch_bits<D, T, 8>(a, stream);
  if (a.bits == 4) return launch_bits<D, T, 4>(a, stream);
  return hipErrorInvalidValue;
}

}  // namespace

hipError_t launch_kv_quant(const KvQuantArgs& a, hipStream_t stream) {
  if (a.d == 64) return a.bf16 ? launch<64, __bf16>(a, stream) : launch<64, float>(a, stream);
  return a.bf16 ? launch<128, __bf16>(a, stream) : launch<128, float>(a, stream);
}

}  // namespace fattn
