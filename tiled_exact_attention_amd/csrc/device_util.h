// Device helpers shared by the gfx950 kernels: vector types, MFMA wrappers,
// transposed LDS reads and packed conversions.
//
// Lane layouts (checked on gfx950 with an in-bounds probe):
//  * v_mfma_f32_32x32x16_bf16: A[i][k] in lane i%32 (i = l%32), k = 8*(l/32)+e;
//    B[k][j] in lane j = l%32, k = 8*(l/32)+e; C[i][j] in lane j = l%32,
//    register r holds row i = 8*(r/4) + 4*(l/32) + r%4.
//  * v_mfma_f32_16x16x32_bf16: A[i][k] in lane i = l%16, k = 8*(l/16)+e;
//    B[k][j] in lane j = l%16, k = 8*(l/16)+e; C[i][j] in lane j = l%16,
//    register r holds row i = 4*(l/16) + r.
//  * ds_read_b64_tr_b16: within each group of 16 lanes, lane t receives
//    element t%4 of the 4-element (8-byte) pieces addressed by lanes
//    t/4 + 4e, e = 0..3.  If lane s of the group addresses row R0 + s/4,
//    columns C0 + 4*(s%4) .. +3 of a row-major 16-bit matrix, lane t gets
//    column C0 + t of rows R0 .. R0+3.
//  * ds_read_b64_tr_b8: within each group of 16 lanes, lane t receives byte
//    t%8 of the 8-byte pieces addressed by lanes 2e + t/8, e = 0..7.  If lane
//    s addresses row rho(s/2), columns C0 + 8*(s%2) .. +7 of a row-major byte
//    matrix, lane t gets column C0 + t of rows rho(0) .. rho(7).
#pragma once

#include <hip/hip_runtime.h>
#include <cstdint>

namespace fattn {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef short i16x4 __attribute__((ext_vector_type(4)));
typedef short i16x8 __attribute__((ext_vector_type(8)));
typedef int i32x2 __attribute__((ext_vector_type(2)));

#define FATTN_LDS(T, p) ((__attribute__((address_space(3))) T*)(p))

// 16-byte loads and stores with the non-temporal hint (the nt bit of
// global_load / global_store_dwordx4): data that is read or written once
// streams past the caches instead of displacing lines that other kernels
// will reuse.  Measured on MI355X in the prefill-then-decode step: the
// decode's cache stream 392 -> 345 us with non-temporal loads, and 345 ->
// 338 us once the prefill also writes its output non-temporally (the
// output's dirty lines no longer come back as write-backs during the decode).
typedef unsigned u32x4 __attribute__((ext_vector_type(4)));
__device__ __forceinline__ void store_nt16(void* p, const uint4& v) {
  __builtin_nontemporal_store(__builtin_bit_cast(u32x4, v), reinterpret_cast<u32x4*>(p));
}
__device__ __forceinline__ uint4 load_nt16(const void* p) {
  return __builtin_bit_cast(uint4, __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(p)));
}
typedef unsigned u32x2 __attribute__((ext_vector_type(2)));
__device__ __forceinline__ void store_nt8(void* p, uint32_t lo, uint32_t hi) {
  __builtin_nontemporal_store(u32x2{lo, hi}, reinterpret_cast<u32x2*>(p));
}
__device__ __forceinline__ void store_nt4(void* p, uint32_t v) {
  __builtin_nontemporal_store(v, reinterpret_cast<uint32_t*>(p));
}

__device__ __forceinline__ f32x16 mfma32(const bf16x8& a, const bf16x8& b, const f32x16& c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
}

__device__ __forceinline__ f32x4 mfma16(const bf16x8& a, const bf16x8& b, const f32x4& c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
}

// Asynchronous 16-byte-per-lane copy HBM -> LDS in buffer form
// (buffer_load_dwordx4 ... lds): lane l's 16 bytes from base + voff land at
// lds_dst + 16*l.  base and lds_dst must be uniform over the wave; voff is per
// lane.  The resource descriptor is raw: stride 0, a record count no byte
// offset below 4 GiB reaches, and word 3 = 0x00020000 (data format 32 bits; a
// zero data format makes gfx9 treat every access as out of range).
// Completion is tracked by vmcnt (wait_vmcnt).
// The flat form (global_load_lds_dwordx4) does the same copy, but while one is
// in flight the compiler assumes any LDS read may alias it (waiting for the
// copies before reads of other buffers) and stops counting LDS reads exactly
// (every LDS wait becomes lgkmcnt(0)); the buffer form keeps both waits exact.
__device__ __forceinline__ void buffer_to_lds16(const void* base, uint32_t voff, void* lds_dst) {
  const __amdgpu_buffer_rsrc_t rsrc =
      __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), 0, 0xffffffff, 0x00020000);
  __builtin_amdgcn_raw_ptr_buffer_load_lds(rsrc, FATTN_LDS(void, lds_dst), 16, voff, 0, 0, 0);
}

// The 4-byte-per-lane copy (buffer_load_dword ... lds): lane l's 4 bytes from
// base + voff land at lds_dst + 4*l.
__device__ __forceinline__ void buffer_to_lds4(const void* base, uint32_t voff, void* lds_dst) {
  const __amdgpu_buffer_rsrc_t rsrc =
      __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), 0, 0xffffffff, 0x00020000);
  __builtin_amdgcn_raw_ptr_buffer_load_lds(rsrc, FATTN_LDS(void, lds_dst), 4, voff, 0, 0, 0);
}

// s_waitcnt vmcnt(N) (gfx9 encoding; expcnt and lgkmcnt left unconstrained).
template <int N>
__device__ __forceinline__ void wait_vmcnt() {
  static_assert(N >= 0 && N < 64, "vmcnt is 6 bits");
  __builtin_amdgcn_s_waitcnt((N & 15) | (7 << 4) | (15 << 8) | ((N >> 4) << 14));
}

// Transposed 16-bit LDS read (see the layout note above); p is an LDS address.
__device__ __forceinline__ i16x4 lds_read_tr16(const void* p) {
  return __builtin_amdgcn_ds_read_tr16_b64_v4i16(FATTN_LDS(i16x4, const_cast<void*>(p)));
}

// Transposed 8-bit LDS read (see the layout note above); p is an LDS address.
__device__ __forceinline__ i32x2 lds_read_tr8(const void* p) {
  return __builtin_amdgcn_ds_read_tr8_b64_v2i32(FATTN_LDS(i32x2, const_cast<void*>(p)));
}

// Round-to-nearest-even fp32 -> bf16 of 8 values.
__device__ __forceinline__ bf16x8 to_bf16x8(float a0, float a1, float a2, float a3,
                                            float a4, float a5, float a6, float a7) {
  bf16x8 r;
  r[0] = (__bf16)a0; r[1] = (__bf16)a1; r[2] = (__bf16)a2; r[3] = (__bf16)a3;
  r[4] = (__bf16)a4; r[5] = (__bf16)a5; r[6] = (__bf16)a6; r[7] = (__bf16)a7;
  return r;
}

// 8 signed bytes (two dwords, byte 0 of lo first) -> 8 bf16 (exact: |x| <= 128).
__device__ __forceinline__ bf16x8 i8x8_to_bf16x8(uint32_t lo, uint32_t hi) {
  return to_bf16x8((float)(int8_t)(lo), (float)(int8_t)(lo >> 8),
                   (float)(int8_t)(lo >> 16), (float)(int8_t)(lo >> 24),
                   (float)(int8_t)(hi), (float)(int8_t)(hi >> 8),
                   (float)(int8_t)(hi >> 16), (float)(int8_t)(hi >> 24));
}

__device__ __forceinline__ i16x8 concat_i16x4(const i16x4& a, const i16x4& b) {
  return __builtin_shufflevector(a, b, 0, 1, 2, 3, 4, 5, 6, 7);
}

// max(x[l], x[l ^ 32]) in every lane l (v_permlane32_swap: no LDS traffic).
__device__ __forceinline__ float max_across_halves(float x) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}

__device__ __forceinline__ float wave_max_xor(float x, int mask) {
  return fmaxf(x, __shfl_xor(x, mask));
}

// LDS swizzle of the bf16 attention kernels' K/V (and Q/dO) tiles, rows of d
// bf16: chunk c (16 bytes) of tile row r is stored at chunk position
// c ^ swz(r).  swz is GF(2)-linear in the low four row bits and chosen (by an
// exhaustive search) so that both read patterns are free of bank conflicts:
// row reads (16 rows at one chunk, the MFMA A operand) and transposed reads
// (4 consecutive rows x 4 chunks, ds_read_b64_tr_b16).
template <int D>
__device__ __forceinline__ int swz(int r) {
  if constexpr (D == 128) {
    return ((r & 1) ? 4 : 0) ^ ((r & 2) ? 10 : 0) ^ ((r & 4) ? 1 : 0) ^ ((r & 8) ? 2 : 0);
  } else {
    return ((r & 1) ? 2 : 0) ^ ((r & 2) ? 4 : 0) ^ ((r & 4) ? 1 : 0) ^ ((r & 8) ? 2 : 0);
  }
}

// Writes one wave's 32 x D output tile as bf16 rows.  The tile is held in the
// accumulator layout of the 32x32 matrix product (lane lq's values are row lq;
// acc[nb][4g + e] is column nb*32 + 8g + 4*(lane/32) + e), each value times
// mul.  The rows go through `stage` (this wave's own 32 * 2D bytes of LDS,
// which no other wave may touch meanwhile) and leave as 16-byte stores of
// whole rows: 4 rows per instruction at D = 128, 8 at D = 64, instead of
// sixteen 8-byte pieces of 32 different rows per lane.  16-byte chunks are
// XOR-swizzled by row so that neither the 8-byte writes (one chunk of 32 rows)
// nor the 16-byte reads (whole rows) conflict in the LDS banks.  The global
// stores carry the non-temporal hint.  Tile row r goes to base + row_off(r)
// bytes, or nowhere if row_off(r) is kSkipRow; base is the same for the whole
// wave and the offsets are 32-bit, so each store addresses a scalar base plus
// a lane offset (measured on MI355X: the d = 64 prefill's epilogue issues
// about a third fewer vector instructions than with a 64-bit address per row).
constexpr uint32_t kSkipRow = 0xffffffffu;
template <int D, class RowOff>
__device__ __forceinline__ void store_tile_rows_bf16(char* stage, const f32x16* acc, float mul, char* base,
                                                     RowOff row_off) {
  constexpr int ROWB = 2 * D, KCH = D / 8, NB = D / 32, RPI = 1024 / ROWB;
  static_assert(D == 64 || D == 128, "head dims of the kernels");
  const int lane = threadIdx.x & 63, lq = lane & 31, hh = lane >> 5;
  auto cswz = [](int r) { return D == 128 ? (r & 15) : ((r >> 1) & 7); };
#pragma unroll
  for (int nb = 0; nb < NB; ++nb) {
#pragma unroll
    for (int g = 0; g < 4; ++g) {
      bf16x4 v;
      v[0] = (__bf16)(acc[nb][4 * g + 0] * mul);
      v[1] = (__bf16)(acc[nb][4 * g + 1] * mul);
      v[2] = (__bf16)(acc[nb][4 * g + 2] * mul);
      v[3] = (__bf16)(acc[nb][4 * g + 3] * mul);
      *reinterpret_cast<bf16x4*>(stage + lq * ROWB + (((4 * nb + g) ^ cswz(lq)) << 4) + 8 * hh) = v;
    }
  }
#pragma unroll
  for (int i = 0; i < 32 / RPI; ++i) {
    const int r = i * RPI + lane / KCH, c = lane % KCH;
    const uint4 v = *reinterpret_cast<const uint4*>(stage + r * ROWB + ((c ^ cswz(r)) << 4));
    const uint32_t off = row_off(r);
    if (off != kSkipRow) store_nt16(base + (off + uint32_t(c) * 16u), v);  // read by a later kernel
  }
}

// Rows and lengths of one sequence: dense batches index b * S; packed batches
// read the cumulative offsets, clamped so that no value can address memory
// outside the packed tensors.  For a packed batch the Sq argument is the
// caller's bound on the query lengths, which sizes the grid only: the
// returned Sq is the sequence's own length, so the causal diagonal (offset
// Skv_b - Sq_b) stays right for a sequence longer than that bound, whose
// rows past the grid are then simply not computed (Skv is unused).
// Unsigned division by a run-time divisor d (1 <= d < 2^31) of a numerator
// below 2^31, as a multiply-high, an add and a shift (the round-up method of
// Granlund and Montgomery, "Division by invariant integers using
// multiplication", 1994): with l = ceil(log2 d) and
// m = floor(2^32 (2^l - d) / d) + 1, a / d = (mulhi(a, m) + a) >> l.  The
// multiplier is formed on the host; on uniform values the quotient stays on
// the scalar unit (a plain division by a kernel argument is expanded through
// the vector unit's reciprocal, per lane).
struct UDiv {
  uint32_t m = 1, l = 0;
  static UDiv make(uint32_t d) {
    UDiv r;
    while ((uint32_t(1) << r.l) < d) ++r.l;
    r.m = uint32_t(((uint64_t(1) << 32) * ((uint64_t(1) << r.l) - d)) / d + 1);
    return r;
  }
  __device__ __forceinline__ uint32_t div(uint32_t a) const { return (__umulhi(a, m) + a) >> l; }
};

struct SeqView {
  int Sq, Skv;
  int64_t q_row0, k_row0;   // first packed row of the sequence
  int64_t lse0, lse_hs;     // lse index of (head 0, position 0), head stride
};

__device__ __forceinline__ SeqView seq_view(const int* cu_q, const int* cu_k, int total_q,
                                            int total_k, int b, int Hq, int Sq, int Skv) {
  SeqView s;
  if (!cu_q) {
    s.Sq = Sq;
    s.Skv = Skv;
    s.q_row0 = int64_t(b) * Sq;
    s.k_row0 = int64_t(b) * Skv;
    s.lse0 = int64_t(b) * Hq * Sq;
    s.lse_hs = Sq;
    return s;
  }
  const int q0 = min(max(cu_q[b], 0), total_q), q1 = min(max(cu_q[b + 1], q0), total_q);
  const int k0 = min(max(cu_k[b], 0), total_k), k1 = min(max(cu_k[b + 1], k0), total_k);
  s.Sq = q1 - q0;
  s.Skv = k1 - k0;
  s.q_row0 = q0;
  s.k_row0 = k0;
  s.lse0 = q0;
  s.lse_hs = total_q;
  return s;
}

}  // namespace fattn
