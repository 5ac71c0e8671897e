// Appending new tokens to the int8 KV cache (the step before int8 decode).
//
// Each (batch, token, kv head) row x of d values becomes d int8 codes and one
// fp32 scale: scale = absmax(x) / 127, code = clamp(rint(x / scale), -127,
// 127) with ties to even, an all-zero row giving scale 0 and zero codes (the
// per-token, per-head symmetric scheme of the int8 cache; [FA-3MOVES] move 3
// names the cache, not a scheme).  The codes decide integers, so the
// arithmetic is exactly the one the cache format is defined by: IEEE fp32
// with correctly rounded divisions (no reciprocal approximation).
//
// gfx950: the kernel is HBM-bound (2 or 4 bytes read and 1 written per
// element).  A row is handled by d/8 consecutive lanes, 8 values each (one
// 16-byte bf16 load or two fp32 loads), the row's absmax reduced with
// cross-lane xor shuffles; each lane stores its 8 codes as one 8-byte write
// into the head-major cache, the row's first lane the scale.
#include "device_util.h"
#include "launch.h"

namespace fattn {
namespace {

constexpr int kThreads = 256;

template <int D, typename T>
__global__ __launch_bounds__(kThreads) void kv_quant_kernel(const T* __restrict__ x,
                                                            int8_t* __restrict__ codes,
                                                            float* __restrict__ scales,
                                                            int64_t rows, int Tn, int Hkv,
                                                            int pos, int cap) {
  constexpr int L = D / 8;                     // lanes per row
  constexpr int RPB = kThreads / L;            // rows per block
  const int lane_in_row = threadIdx.x % L;
  const int64_t r = int64_t(blockIdx.x) * RPB + threadIdx.x / L;  // row = (b, t, h)
  const bool live = r < rows;
  const int64_t rr = live ? r : 0;
  const int h = int(rr % Hkv);
  const int64_t bt = rr / Hkv;
  const int t = int(bt % Tn);
  const int64_t b = bt / Tn;

  float v[8];
  const T* src = x + rr * D + 8 * lane_in_row;
  if constexpr (sizeof(T) == 2) {
    const bf16x8 raw = *reinterpret_cast<const bf16x8*>(src);
#pragma unroll
    for (int e = 0; e < 8; ++e) v[e] = float(raw[e]);
  } else {
    const f32x4 a = *reinterpret_cast<const f32x4*>(src);
    const f32x4 c = *reinterpret_cast<const f32x4*>(src + 4);
#pragma unroll
    for (int e = 0; e < 4; ++e) { v[e] = a[e]; v[4 + e] = c[e]; }
  }
  float amax = 0.f;
#pragma unroll
  for (int e = 0; e < 8; ++e) amax = fmaxf(amax, fabsf(v[e]));
#pragma unroll
  for (int m = 1; m < L; m <<= 1) amax = fmaxf(amax, __shfl_xor(amax, m));
  const float scale = amax / 127.0f;

  uint32_t lo = 0, hi = 0;
#pragma unroll
  for (int e = 0; e < 8; ++e) {
    float q = 0.f;
    if (scale != 0.f) {
      q = __builtin_rintf(v[e] / scale);
      q = fminf(fmaxf(q, -127.f), 127.f);
    }
    const uint32_t byte = uint32_t(int32_t(q)) & 0xffu;
    if (e < 4) lo |= byte << (8 * e); else hi |= byte << (8 * (e - 4));
  }
  if (!live) return;
  const int64_t slot = (b * Hkv + h) * int64_t(cap) + pos + t;
  *reinterpret_cast<uint2*>(codes + slot * D + 8 * lane_in_row) = make_uint2(lo, hi);
  if (lane_in_row == 0) scales[slot] = scale;
}

template <int D, typename T>
hipError_t launch(const KvQuantArgs& a, hipStream_t stream) {
  constexpr int RPB = kThreads / (D / 8);
  const int64_t rows = int64_t(a.B) * a.T * a.Hkv;
  const int64_t blocks = (rows + RPB - 1) / RPB;
  if (blocks > 0x7fffffff) return hipErrorInvalidConfiguration;
  hipLaunchKernelGGL((kv_quant_kernel<D, T>), dim3(unsigned(blocks)), dim3(kThreads), 0, stream,
                     static_cast<const T*>(a.x), a.codes, a.scales, rows, a.T, a.Hkv, a.pos, a.cap);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_kv_quant(const KvQuantArgs& a, hipStream_t stream) {
  if (a.d == 64) return a.bf16 ? launch<64, __bf16>(a, stream) : launch<64, float>(a, stream);
  return a.bf16 ? launch<128, __bf16>(a, stream) : launch<128, float>(a, stream);
}

}  // namespace fattn
