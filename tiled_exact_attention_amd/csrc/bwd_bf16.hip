// Backward pass of bf16 tiled exact attention on the gfx950 matrix cores.
//
// Method ([FA-NPU] recomputation section: the backward pass recomputes the
// attention weights from the row statistics saved by the forward instead of
// storing them): with the forward's lse, a tile's probabilities are
// P = exp(scale q.k - lse), recomputed tile by tile, and
//   dV = P^T dO,  dP = dO V^T,  D = rowsum(dO * O),  dS = P (dP - D),
//   dQ = scale dS K,  dK = scale dS^T Q,
// the gradients of the forward's definition (D equals rowsum(P * dP) because
// O = P V).  Nothing of size S x S reaches HBM.
//
// Two kernels (three for split groups) on the caller's stream:
//  * bwd_dq_kernel: the forward's layout (4 waves x 32 query rows, GQA head
//    chunks, K/V tiles of 64 keys streamed HBM -> LDS by LDS-DMA into the
//    swizzled layout).  Each wave first forms D and lse * log2(e) of its rows
//    (from its dO rows and O) and writes them to the workspace; a row with no
//    visible key gets +inf, so its recomputed probabilities are exactly 0.
//    Per tile S^T = K Q^T and dP^T = V dO^T (A = K / V rows from LDS, B = the
//    wave's Q / dO rows held in registers); dS^T lands in the B-operand
//    layout; dQ^T += K^T dS^T with K^T from transposed LDS reads.  No running
//    max: lse is known.
//  * bwd_dkdv_kernel: 4 waves x 32 keys, K and V rows in registers as B
//    operands; query tiles of 64 rows (Q, dO, lse, D) stream through LDS for
//    every query head of (a split of) the kv head's group and every tile that
//    sees the block's keys.  S = Q K^T and dP = dO V^T put one key per lane,
//    which is the B layout of dV^T += dO^T P and dK^T += Q^T dS (dO^T / Q^T
//    from transposed LDS reads).  The sum over query heads stays in
//    registers; when the grid would be too small (few kv heads, many query
//    heads: MQA) the group is split across blocks that write fp32 partials,
//    and bwd_reduce_kernel adds them in split order.  No atomics: the result
//    does not depend on scheduling.
// P and dS are rounded to bf16 for their products; accumulation is fp32.
#include "device_util.h"
#include "launch.h"

#include <cmath>
#include <type_traits>

namespace fattn {
namespace {

// LDS operand reads are issued this many matrix products ahead of their use
// (dK/dV kernel; the dQ kernel, at two waves per SIMD, has fewer registers).
constexpr int kLA = 3;
constexpr int kLAq = 2;

// sched_group_barrier sequences: N instructions of class M (0x008 matrix
// product, 0x100 LDS read), or REP repetitions of (N1 of M1, N2 of M2).
// f(integral_constant<int, 0>), ..., f(integral_constant<int, N-1>), in order.
template <int N, typename Fn>
__device__ __forceinline__ void static_for(Fn&& f) {
  if constexpr (N > 0) {
    static_for<N - 1>(f);
    f(std::integral_constant<int, N - 1>{});
  }
}
template <int M, int N>
__device__ __forceinline__ void sched_group() {
  if constexpr (N > 0) __builtin_amdgcn_sched_group_barrier(M, N, 0);
}
template <int M1, int N1, int M2, int N2, int REP>
__device__ __forceinline__ void sched_pairs() {
  if constexpr (REP > 0) {
    __builtin_amdgcn_sched_group_barrier(M1, N1, 0);
    __builtin_amdgcn_sched_group_barrier(M2, N2, 0);
    sched_pairs<M1, N1, M2, N2, REP - 1>();
  }
}

constexpr int kWaves = 4;
constexpr int kThreads = 64 * kWaves;
constexpr int kBM = 32 * kWaves;  // query rows per dQ block
constexpr int kBN = 64;           // keys per dQ tile
constexpr int kBK = 32 * kWaves;  // keys per dK/dV block
constexpr int kBQ = 64;           // query rows per dK/dV tile
constexpr float kLog2e = 1.4426950408889634f;

struct BwdParams {
  const __bf16* q;
  const __bf16* k;
  const __bf16* v;
  const __bf16* o;
  const __bf16* dout;
  const float* lse;
  __bf16* dq;
  __bf16* dk;
  __bf16* dv;
  float* l2;   // workspace [B, Hq, Sq]: lse * log2(e), +inf for a row with no key (written by the dQ kernel)
  float* dd;   // workspace [B, Hq, Sq]: D = rowsum(dO * O) (written by the dQ kernel)
  float* part_k;  // workspace [nsplit, B, Skv, Hkv, d] fp32 partial dK (nsplit > 1)
  float* part_v;  // ... and dV
  int nsplit;     // query-head splits of a kv head's group in the dK/dV kernel
  int hps;        // query heads per split
  int B, Hq, Hkv, Sq, Skv;
  int G;         // query heads per kv head
  int gc_shift;  // log2 of the heads per dQ row chunk
  int nchunk;    // G / GC
  int nqb;       // dQ row blocks per (b, kv head, head chunk)
  int nx;        // B * Hkv * nchunk
  UDiv div_nx, div_nchunk, div_hkv, div_nbh, div_nsplit;  // dividers of the block mappings
  float c;       // |scale| * log2(e), >= 1e-30
  float scale;   // the signed scale
  int negate;    // 1 if scale < 0 (Q, or K, sign flipped on load)
  int causal, window;
};

// ------------------------------------------------------------------------ dQ
template <int D>
__global__ __launch_bounds__(kThreads, 2) void bwd_dq_kernel(BwdParams p) {
  constexpr int KCH = D / 8;                 // 16-byte chunks per K/V row
  constexpr int ROWB = D * 2;                // bytes per K/V row
  constexpr int TILE_B = kBN * ROWB;         // bytes of one K (or V) tile
  constexpr int STAGE_B = 2 * TILE_B;        // K tile then V tile
  constexpr int LPI = 1024 / ROWB;           // rows filled by one 1 KB LDS-DMA instruction
  constexpr int NLD = kBN / (kWaves * LPI);  // LDS-DMA instructions per wave per tensor per tile
  constexpr int KSTEPS = D / 16;             // k-steps of the head-dim products
  constexpr int NB = D / 32;                 // 32-wide blocks of a row
  static_assert(NLD * LPI * kWaves == kBN, "tile rows must split evenly over the waves");
  __shared__ __attribute__((aligned(1024))) char lds[2 * STAGE_B];

  // ---- block -> (batch, kv head, head chunk, query block); heavy blocks first
  const int id = blockIdx.x;
  const int slot = int(p.div_nx.div(uint32_t(id)));
  const int x = id - slot * p.nx;
  const int qb = p.causal ? p.nqb - 1 - slot : slot;
  const int xc = int(p.div_nchunk.div(uint32_t(x)));
  const int chunk = x - xc * p.nchunk;
  const int b = int(p.div_hkv.div(uint32_t(xc)));
  const int hk = xc - b * p.Hkv;
  const int gc = 1 << p.gc_shift;
  const int rows_pos = kBM >> p.gc_shift;
  const int p0 = qb * rows_pos;
  const int hq0 = hk * p.G + chunk * gc;
  const int Sq = p.Sq, Skv = p.Skv;

  const int lane = threadIdx.x & 63;
  const int w = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int lq = lane & 31;
  const int hh = lane >> 5;
  const int row = w * 32 + lq;
  const int pos = p0 + (row >> p.gc_shift);
  const int hq = hq0 + (row & (gc - 1));
  const bool row_ok = pos < Sq;
  const int64_t off = int64_t(Skv) - Sq;

  // ---- key ranges: block band [jb, je); this row's visible keys [row_lo, row_hi)
  const int bpos_hi = min(p0 + rows_pos - 1, Sq - 1);
  int64_t jb = 0, je = Skv;
  int64_t row_lo = 0, row_hi = Skv;
  const int wpos_lo = p0 + ((w * 32) >> p.gc_shift);
  const int wpos_hi = min(p0 + ((w * 32 + 31) >> p.gc_shift), Sq - 1);
  // the bounds rise with the row: over the wave's rows row_hi runs from
  // w_hi_min to w_hi_max and row_lo from w_lo_min to w_lo_max (w_lo_max from
  // the last row even past Sq, as row_lo is for such rows)
  const int wpos_end = p0 + ((w * 32 + 31) >> p.gc_shift);
  int64_t w_hi_max = Skv, w_lo_min = 0, w_hi_min = Skv, w_lo_max = 0;
  if (p.causal) {
    je = min(int64_t(Skv), bpos_hi + off + 1);
    row_hi = min(int64_t(Skv), pos + off + 1);
    w_hi_max = min(int64_t(Skv), wpos_hi + off + 1);
    w_hi_min = min(int64_t(Skv), wpos_lo + off + 1);
    if (p.window > 0) {
      jb = max(int64_t(0), p0 + off - p.window + 1);
      row_lo = max(int64_t(0), pos + off - p.window + 1);
      w_lo_min = max(int64_t(0), wpos_lo + off - p.window + 1);
      w_lo_max = max(int64_t(0), wpos_end + off - p.window + 1);
    }
  }
  const bool wave_active = wpos_lo < Sq;
  const int ntiles = je > jb ? int((je - jb + kBN - 1) / kBN) : 0;

  // ---- Q (sign-flipped for a negative scale) and dO rows as B operands
  // (k-step m: columns 16m + 8hh .. +7); lse2 and D of this lane's row
  bf16x8 qf[KSTEPS], df[KSTEPS];
  {
    const int64_t ro = ((int64_t(b) * Sq + (row_ok ? pos : 0)) * p.Hq + hq) * D;
#pragma unroll
    for (int m = 0; m < KSTEPS; ++m) {
      uint4 raw = *reinterpret_cast<const uint4*>(p.q + ro + 16 * m + 8 * hh);
      if (p.negate) {
        raw.x ^= 0x80008000u; raw.y ^= 0x80008000u; raw.z ^= 0x80008000u; raw.w ^= 0x80008000u;
      }
      qf[m] = __builtin_bit_cast(bf16x8, raw);
      df[m] = *reinterpret_cast<const bf16x8*>(p.dout + ro + 16 * m + 8 * hh);
    }
  }
  // D = rowsum(dO * O) and lse2 = lse * log2(e) (+inf for a row that sees no
  // key) of this lane's row; the dK/dV kernel reads them from the workspace.
  // Each 8-value chunk is an fma chain from 0 and the chunk sums are added as a
  // balanced tree (pairs of neighbouring chunks first); this lane holds chunks
  // 2m + hh, its partner lane ^ 32 the others.
  const int64_t srow = (int64_t(b) * p.Hq + hq) * Sq + (row_ok ? pos : 0);
  float l2, dd;
  {
    const int64_t ro = ((int64_t(b) * Sq + (row_ok ? pos : 0)) * p.Hq + hq) * D;
    float c[KSTEPS];
#pragma unroll
    for (int m = 0; m < KSTEPS; ++m) {
      const bf16x8 o8 = *reinterpret_cast<const bf16x8*>(p.o + ro + 16 * m + 8 * hh);
      c[m] = 0.f;
#pragma unroll
      for (int e = 0; e < 8; ++e) c[m] = fmaf(float(o8[e]), float(df[m][e]), c[m]);
      c[m] += __shfl_xor(c[m], 32);  // chunks 2m and 2m + 1
    }
#pragma unroll
    for (int span = 1; span < KSTEPS; span <<= 1) {
#pragma unroll
      for (int m = 0; m < KSTEPS; m += 2 * span) c[m] += c[m + span];
    }
    const float lse = row_ok ? p.lse[srow] : -INFINITY;
    l2 = lse == -INFINITY ? INFINITY : lse * kLog2e;
    dd = row_ok ? c[0] : 0.f;
    if (hh == 0 && row_ok) {
      p.dd[srow] = dd;
      p.l2[srow] = l2;
    }
  }

  // ---- LDS read offsets (as the forward): row reads of K and V (A operands
  // of S^T and dP^T), transposed reads of K (A operand of dQ^T = K^T dS^T)
  int koff[KSTEPS];
#pragma unroll
  for (int m = 0; m < KSTEPS; ++m) koff[m] = lq * ROWB + (((2 * m + hh) ^ swz<D>(lq)) << 4);
  const int g16 = lane >> 4, s16 = lane & 15;
  const int h2 = g16 >> 1, nh = g16 & 1;
  int toff[NB][2];
#pragma unroll
  for (int nb = 0; nb < NB; ++nb) {
#pragma unroll
    for (int R = 0; R < 2; ++R) {
      const int r = 4 * h2 + (s16 >> 2) + 8 * R;
      const int col = nb * 32 + nh * 16 + 4 * (s16 & 3);
      toff[nb][R] = r * ROWB + (((col >> 3) ^ swz<D>(r)) << 4) + (col & 7) * 2;
    }
  }

  // ---- LDS-DMA load assignment (as the forward)
  const int64_t kv_stride = int64_t(p.Hkv) * D;
  const __bf16* kbase = p.k + (int64_t(b) * Skv * p.Hkv + hk) * D;
  const __bf16* vbase = p.v + (int64_t(b) * Skv * p.Hkv + hk) * D;
  // (source offsets are recomputed per tile rather than kept in registers)
  auto issue_loads = [&](int64_t j0, char* stage) __attribute__((always_inline)) {
    const __bf16* kt = kbase + j0 * kv_stride;
    const __bf16* vt = vbase + j0 * kv_stride;
    // at d = 128 the lane terms are recomputed here, not held across the
    // loop (held, they spill at 256 registers); at d = 64 holding them is
    // faster
    int ln = lane;
    if constexpr (D >= 128) asm volatile("" : "+v"(ln));
#pragma unroll
    for (int i = 0; i < NLD; ++i) {
      const int r = 16 * w + LPI * i + ln / KCH;
      // rows past the end of the keys re-read the last row
      const int jr = int(min(j0 + r, int64_t(Skv) - 1) - j0);
      const uint32_t e = (uint32_t(jr) * uint32_t(kv_stride) + ((ln % KCH) ^ swz<D>(r)) * 8) * 2u;
      char* dst = stage + (16 * w + LPI * i) * ROWB;
      buffer_to_lds16(kt, e, dst);
      buffer_to_lds16(vt, e, dst + TILE_B);
    }
  };

  f32x16 acc[NB];
#pragma unroll
  for (int nb = 0; nb < NB; ++nb) acc[nb] = f32x16{};

  // Order chosen for register pressure (two waves per SIMD): S^T, then P^T
  // packed to bf16 (the scores die), then dP^T, then dS^T.
  auto compute = [&](int64_t j0, const char* stage, auto masked) __attribute__((always_inline)) {
    // S^T = K Q^T: the two 32-key chains interleaved, operand reads 2*kLAq
    // products ahead (sched_group_barrier: 0x100 = LDS read, 0x008 = product)
    __builtin_amdgcn_s_setprio(1);
    f32x16 s[2];
    {
      bf16x8 ka[KSTEPS][2];
#pragma unroll
      for (int m = 0; m < KSTEPS; ++m)
#pragma unroll
        for (int kb = 0; kb < 2; ++kb) ka[m][kb] = *reinterpret_cast<const bf16x8*>(stage + koff[m] + kb * 32 * ROWB);
      s[0] = f32x16{};
      s[1] = f32x16{};
#pragma unroll
      for (int m = 0; m < KSTEPS; ++m)
#pragma unroll
        for (int kb = 0; kb < 2; ++kb) s[kb] = mfma32(ka[m][kb], qf[m], s[kb]);
      sched_group<0x100, 2 * kLAq>();
      sched_pairs<0x008, 1, 0x100, 1, 2 * KSTEPS - 2 * kLAq>();
      sched_group<0x008, 2 * kLAq>();
    }
    __builtin_amdgcn_s_setprio(0);
    if constexpr (decltype(masked)::value) {
      // per 32-key block, only where an edge cuts it for some row of the wave
      // (scalar tests on the wave's lowest row_hi and highest row_lo), one
      // compare and select per element and edge, each an in-place if-then
#pragma unroll
      for (int kb = 0; kb < 2; ++kb) {
        const int64_t b0 = j0 + 32 * kb;  // first key of the block
        if (w_hi_min < b0 + 32) {
          const int hi = int(row_hi - b0) - 4 * hh;
#pragma unroll
          for (int r = 0; r < 16; ++r) {
            const int kc0 = 8 * (r >> 2) + (r & 3);
            if (kc0 >= hi) s[kb][r] = -INFINITY;
          }
        }
        if (w_lo_max > b0) {
          const int lo = int(row_lo - b0) - 4 * hh;
#pragma unroll
          for (int r = 0; r < 16; ++r) {
            const int kc0 = 8 * (r >> 2) + (r & 3);
            if (kc0 < lo) s[kb][r] = -INFINITY;
          }
        }
      }
    }
    // P^T = 2^(s c - lse2).  This kernel has no product with P: at d = 128 P
    // stays in s in fp32 and dS below is formed from those values; at d = 64
    // P is kept packed in bf16 (16 registers instead of 32, which keeps that
    // kernel at three waves per SIMD) and widened back for dS
    bf16x8 pf[4];
    if constexpr (D >= 128) {
#pragma unroll
      for (int kb = 0; kb < 2; ++kb) {
#pragma unroll
        for (int r = 0; r < 16; ++r) s[kb][r] = __builtin_amdgcn_exp2f(fmaf(s[kb][r], p.c, -l2));
      }
    } else {
#pragma unroll
      for (int kc = 0; kc < 4; ++kc) {
        float e[8];
#pragma unroll
        for (int i = 0; i < 8; ++i) e[i] = __builtin_amdgcn_exp2f(fmaf(s[kc >> 1][8 * (kc & 1) + i], p.c, -l2));
        pf[kc] = to_bf16x8(e[0], e[1], e[2], e[3], e[4], e[5], e[6], e[7]);
      }
    }
    // dP^T = V dO^T, then dS^T = P^T (dP^T - D)
    __builtin_amdgcn_sched_barrier(0);
    __builtin_amdgcn_s_setprio(1);
    f32x16 dp[2];
    {
      bf16x8 va[KSTEPS][2];
#pragma unroll
      for (int m = 0; m < KSTEPS; ++m)
#pragma unroll
        for (int kb = 0; kb < 2; ++kb) va[m][kb] = *reinterpret_cast<const bf16x8*>(stage + TILE_B + koff[m] + kb * 32 * ROWB);
      dp[0] = f32x16{};
      dp[1] = f32x16{};
#pragma unroll
      for (int m = 0; m < KSTEPS; ++m)
#pragma unroll
        for (int kb = 0; kb < 2; ++kb) dp[kb] = mfma32(va[m][kb], df[m], dp[kb]);
      sched_group<0x100, 2 * kLAq>();
      sched_pairs<0x008, 1, 0x100, 1, 2 * KSTEPS - 2 * kLAq>();
      sched_group<0x008, 2 * kLAq>();
    }
    __builtin_amdgcn_sched_barrier(0);
    __builtin_amdgcn_s_setprio(0);
    bf16x8 dsf[4];
#pragma unroll
    for (int kc = 0; kc < 4; ++kc) {
      float e[8];
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        float pv;
        if constexpr (D >= 128) {
          pv = s[kc >> 1][8 * (kc & 1) + i];
        } else {
          // element i of pf[kc] widened to fp32 from its packed dword
          const uint32_t pw = __builtin_bit_cast(u32x4, pf[kc])[i / 2];
          pv = __builtin_bit_cast(float, (i & 1) ? (pw & 0xffff0000u) : (pw << 16));
        }
        e[i] = pv * (dp[kc >> 1][8 * (kc & 1) + i] - dd);
      }
      dsf[kc] = to_bf16x8(e[0], e[1], e[2], e[3], e[4], e[5], e[6], e[7]);
    }
    __builtin_amdgcn_s_setprio(1);
#pragma unroll
    for (int kc = 0; kc < 4; ++kc) {
#pragma unroll
      for (int nb = 0; nb < NB; ++nb) {
        const i16x4 a0 = lds_read_tr16(stage + toff[nb][0] + kc * 16 * ROWB);
        const i16x4 a1 = lds_read_tr16(stage + toff[nb][1] + kc * 16 * ROWB);
        acc[nb] = mfma32(__builtin_bit_cast(bf16x8, concat_i16x4(a0, a1)), dsf[kc], acc[nb]);
      }
    }
    __builtin_amdgcn_s_setprio(0);
  };

  auto step = [&](int t, char* cur, char* nxt, auto masked) __attribute__((always_inline)) {
    wait_vmcnt<0>();
    __syncthreads();
    if (t + 1 < ntiles) issue_loads(jb + int64_t(t + 1) * kBN, nxt);
    const int64_t j0 = jb + int64_t(t) * kBN;
    if constexpr (decltype(masked)::value) {
      if (wave_active && j0 < w_hi_max && j0 + kBN > w_lo_min) compute(j0, cur, masked);
    } else {
      if (wave_active) compute(j0, cur, masked);
    }
  };
  auto pair = [&](int t, auto masked) __attribute__((always_inline)) {
    step(t, lds, lds + STAGE_B, masked);
    if (t + 1 < ntiles) step(t + 1, lds + STAGE_B, lds, masked);
  };
  int t_lo = 0, t_hi = ntiles;
  {
    const int64_t hi_min = p.causal ? min(int64_t(Skv), p0 + off + 1) : int64_t(Skv);
    const int64_t lo_max = (p.causal && p.window > 0) ? max(int64_t(0), bpos_hi + off - p.window + 1) : 0;
    t_hi = hi_min - jb >= kBN ? int(min(int64_t(ntiles), (hi_min - jb) / kBN)) : 0;
    t_lo = lo_max > jb ? int(min(int64_t(t_hi), (lo_max - jb + kBN - 1) / kBN)) : 0;
    t_lo = (t_lo + 1) & ~1;
    t_hi = t_hi > t_lo ? t_lo + ((t_hi - t_lo) & ~1) : t_lo;
  }
  if (ntiles > 0) issue_loads(jb, lds);
  int t = 0;
  for (; t < t_lo; t += 2) pair(t, std::true_type{});
  for (; t < t_hi; t += 2) pair(t, std::false_type{});
  for (; t < ntiles; t += 2) pair(t, std::true_type{});

  // ---- dQ = scale * (K^T dS^T)^T, bf16 (RNE), written as whole rows through
  // the stage the last step did not read (idle once that step's barrier has
  // passed; each wave uses its own quarter)
  char* qbase = reinterpret_cast<char*>(p.dq + ((int64_t(b) * Sq + p0) * p.Hq + hq0) * D);
  store_tile_rows_bf16<D>(lds + (ntiles & 1) * STAGE_B + w * 32 * ROWB, acc, p.scale, qbase,
                          [&](int r) -> uint32_t {
                            const int prow = w * 32 + r;
                            const int dpos = prow >> p.gc_shift;
                            return p0 + dpos < Sq
                                       ? uint32_t(dpos * p.Hq + (prow & (gc - 1))) * uint32_t(2 * D)
                                       : kSkipRow;
                          });
}

// --------------------------------------------------------------------- dK, dV
template <int D>
__global__ __launch_bounds__(kThreads, 1) void bwd_dkdv_kernel(BwdParams p) {
  constexpr int KCH = D / 8;
  constexpr int ROWB = D * 2;
  constexpr int TILE_B = kBQ * ROWB;            // one Q (or dO) tile
  constexpr int STAGE_B = 2 * TILE_B + 2 * kBQ * 4;  // Q, dO, lse2[64], D[64]
  constexpr int LPI = 1024 / ROWB;
  constexpr int NLD = kBQ / (kWaves * LPI);
  constexpr int KSTEPS = D / 16;
  constexpr int NB = D / 32;
  static_assert(NLD * LPI * kWaves == kBQ, "tile rows must split evenly over the waves");
  static_assert(STAGE_B % 256 == 0, "stages start on a bank-period boundary");
  __shared__ __attribute__((aligned(1024))) char lds[2 * STAGE_B];

  // ---- block -> (batch, kv head, head split, key block); for causal masks
  // the early key blocks see the most queries, so they come first.  (An
  // XCD-major order, each XCD taking one (batch, kv head, split) at a time
  // with all its key blocks, cut the kernel's HBM reads on the MHA workload
  // from 735 to 309 MB but was 1-2% slower; the kernel is not bound by HBM.)
  const int nbh = p.B * p.Hkv * p.nsplit;
  const int kbi = int(p.div_nbh.div(blockIdx.x));
  const int x = int(blockIdx.x) - kbi * nbh;
  const int xs = int(p.div_nsplit.div(uint32_t(x)));
  const int split = x - xs * p.nsplit;
  const int b = int(p.div_hkv.div(uint32_t(xs)));
  const int hk = xs - b * p.Hkv;
  const int g0 = split * p.hps;                    // first query head (in the group) of the split
  const int ng = min(p.hps, p.G - g0);             // heads of this split
  const int Sq = p.Sq, Skv = p.Skv;
  const int64_t off = int64_t(Skv) - Sq;
  const int j0 = kbi * kBK;
  const int j1 = min(j0 + kBK, Skv);

  const int lane = threadIdx.x & 63;
  const int w = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int lq = lane & 31;
  const int hh = lane >> 5;
  const int jw = j0 + 32 * w;            // this wave's first key
  const int jwe = min(jw + 32, Skv);     // ... and one past its last
  const int key = jw + lq;
  const bool key_ok = key < Skv;

  // ---- K (sign-flipped for a negative scale) and V rows of this lane's key
  // as B operands (k-step m: columns 16m + 8hh .. +7)
  bf16x8 kf[KSTEPS], vf[KSTEPS];
  {
    const int64_t ro = ((int64_t(b) * Skv + min(key, Skv - 1)) * p.Hkv + hk) * D;
#pragma unroll
    for (int m = 0; m < KSTEPS; ++m) {
      uint4 raw = *reinterpret_cast<const uint4*>(p.k + ro + 16 * m + 8 * hh);
      if (p.negate) {
        raw.x ^= 0x80008000u; raw.y ^= 0x80008000u; raw.z ^= 0x80008000u; raw.w ^= 0x80008000u;
      }
      kf[m] = __builtin_bit_cast(bf16x8, raw);
      vf[m] = *reinterpret_cast<const bf16x8*>(p.v + ro + 16 * m + 8 * hh);
    }
  }

  // ---- query rows that see some key of the block: key j is visible to query
  // i iff j <= i + off (causal) and j > i + off - W (window)
  int i_lo = 0, i_hi = Sq;
  if (p.causal) {
    i_lo = int(max(int64_t(0), int64_t(j0) - off));
    if (p.window > 0) i_hi = int(min(int64_t(Sq), int64_t(j1) - 1 - off + p.window));
  }
  const int tq0 = i_lo / kBQ;
  const int ntq = i_hi > i_lo ? (i_hi + kBQ - 1) / kBQ - tq0 : 0;
  const int niter = ng > 0 ? ntq * ng : 0;  // (query head of the split, query tile), head-major

  // ---- LDS offsets: row reads of Q / dO (A operands of S and dP),
  // transposed reads of dO / Q (A operands of dV^T and dK^T)
  int koff[KSTEPS];
#pragma unroll
  for (int m = 0; m < KSTEPS; ++m) koff[m] = lq * ROWB + (((2 * m + hh) ^ swz<D>(lq)) << 4);
  const int g16 = lane >> 4, s16 = lane & 15;
  const int h2 = g16 >> 1, nh = g16 & 1;
  int toff[NB][2];
#pragma unroll
  for (int nb = 0; nb < NB; ++nb) {
#pragma unroll
    for (int R = 0; R < 2; ++R) {
      const int r = 4 * h2 + (s16 >> 2) + 8 * R;
      const int col = nb * 32 + nh * 16 + 4 * (s16 & 3);
      toff[nb][R] = r * ROWB + (((col >> 3) ^ swz<D>(r)) << 4) + (col & 7) * 2;
    }
  }

  // ---- LDS-DMA loads of one (head, query tile): wave w fills rows
  // 16w .. 16w+15 of the Q and dO tiles; waves 0 and 1 also fetch the 64
  // lse2 and D values
  const int64_t q_stride = int64_t(p.Hq) * D;
  uint32_t goff[NLD];  // element offsets within a tile (below 2^31: Hq * d < 2^24)
  int ld_row[NLD];
#pragma unroll
  for (int i = 0; i < NLD; ++i) {
    const int r = 16 * w + LPI * i + lane / KCH;
    ld_row[i] = r;
    goff[i] = uint32_t(r) * uint32_t(q_stride) + ((lane % KCH) ^ swz<D>(r)) * 8;
  }
  auto issue_loads = [&](int g, int i0, char* stage) __attribute__((always_inline)) {
    const int hq = hk * p.G + g;
    const __bf16* qb = p.q + (int64_t(b) * Sq * p.Hq + hq) * D;
    const __bf16* db = p.dout + (int64_t(b) * Sq * p.Hq + hq) * D;
    const __bf16* qt = qb + int64_t(i0) * q_stride;
    const __bf16* dt = db + int64_t(i0) * q_stride;
    if (i0 + kBQ <= Sq) {
#pragma unroll
      for (int i = 0; i < NLD; ++i) {
        char* dst = stage + (16 * w + LPI * i) * ROWB;
        buffer_to_lds16(qt, goff[i] * 2u, dst);
        buffer_to_lds16(dt, goff[i] * 2u, dst + TILE_B);
      }
    } else {
      // last tile of the queries: rows past the end re-read the last row
#pragma unroll
      for (int i = 0; i < NLD; ++i) {
        const int back = max(i0 + ld_row[i] - (Sq - 1), 0);
        const uint32_t e = (goff[i] - uint32_t(back) * uint32_t(q_stride)) * 2u;
        char* dst = stage + (16 * w + LPI * i) * ROWB;
        buffer_to_lds16(qt, e, dst);
        buffer_to_lds16(dt, e, dst + TILE_B);
      }
    }
    if (w < 2) {
      const float* src = (w == 0 ? p.l2 : p.dd) + (int64_t(b) * p.Hq + hq) * Sq + i0;
      buffer_to_lds4(src, uint32_t(min(lane, Sq - 1 - i0)) * 4u, stage + 2 * TILE_B + w * (kBQ * 4));
    }
  };

  f32x16 acck[NB], accv[NB];
#pragma unroll
  for (int nb = 0; nb < NB; ++nb) {
    acck[nb] = f32x16{};
    accv[nb] = f32x16{};
  }

  // One (head, query tile) for this wave's 32 keys.  Registers r of query
  // half qh hold query row i0 + 32qh + 8(r/4) + 4hh + r%4 (the C layout of
  // S = Q K^T with one key per lane).
  //
  // The tile's matrix products run in four phases, one product per step:
  // S = Q K^T and dP = dO V^T (2 KSTEPS each; Q / dO row reads from LDS),
  // then dV^T += dO^T P and dK^T += Q^T dS (4 NB each; transposed dO / Q
  // reads).  Each step also issues the operand reads of the product kLA
  // ahead.  With one wave per SIMD no other wave covers the vector work, so
  // it is spread over products that do not depend on it: P = 2^(s c - lse2)
  // over the dP steps, dS = P (dP - D) over the dV steps, a few elements per
  // step.  Each slice is pinned into its step by empty asm operands (the
  // sched_barrier fences order the machine scheduler, not IR-level code
  // motion).  dS is formed from the bf16 P of the dV products (so dK and dV
  // use the same P) and overwrites dP in place.
  auto compute = [&](int i0, const char* stage, auto masked) __attribute__((always_inline)) {
    constexpr int NS = 2 * KSTEPS;       // products of S, and of dP
    constexpr int NT = 4 * NB;           // products of dV, and of dK
    constexpr int NPR = 2 * NS + 2 * NT;
    constexpr int EP = 32 / NS;          // P elements per dP step
    constexpr int ES = 32 / NT;          // dS elements per dV step
    static_assert(EP * NS == 32 && ES * NT == 32, "elements split evenly over the steps");
    const float* l2s = reinterpret_cast<const float*>(stage + 2 * TILE_B);
    const float* dds = l2s + kBQ;
    f32x16 s[2], dp[2];
    bf16x8 ra[NPR];    // row operand reads (S, dP products)
    i16x4 ta[NPR][2];  // transposed operand reads (dV, dK products)
    auto read = [&](auto I) __attribute__((always_inline)) {
      constexpr int i = decltype(I)::value;
      if constexpr (i < 2 * NS) {
        constexpr int k = i % NS, m = k / 2, qh = k % 2, src = i < NS ? 0 : TILE_B;
        ra[i] = *reinterpret_cast<const bf16x8*>(stage + src + koff[m] + qh * 32 * ROWB);
      } else {
        constexpr int k = (i - 2 * NS) % NT, kc = k / NB, nb = k % NB;
        constexpr int src = i < 2 * NS + NT ? TILE_B : 0;
        ta[i][0] = lds_read_tr16(stage + src + toff[nb][0] + kc * 16 * ROWB);
        ta[i][1] = lds_read_tr16(stage + src + toff[nb][1] + kc * 16 * ROWB);
      }
    };
    bf16x8 pf[4], dsf[4];  // P and dS as B operands (k-step kc: registers 8(kc&1) .. +7 of half kc/2)
    auto product = [&](auto I) __attribute__((always_inline)) {
      constexpr int i = decltype(I)::value;
      if constexpr (i < NS) {
        s[i % 2] = mfma32(ra[i], kf[i / 2], s[i % 2]);
      } else if constexpr (i < 2 * NS) {
        dp[i % 2] = mfma32(ra[i], vf[(i - NS) / 2], dp[i % 2]);
      } else {
        constexpr int k = (i - 2 * NS) % NT, kc = k / NB, nb = k % NB;
        const bf16x8 a = __builtin_bit_cast(bf16x8, concat_i16x4(ta[i][0], ta[i][1]));
        if constexpr (i < 2 * NS + NT) {
          accv[nb] = mfma32(a, pf[kc], accv[nb]);
        } else {
          acck[nb] = mfma32(a, dsf[kc], acck[nb]);
        }
      }
    };
    // lse2 and D of this lane's rows, group g = rows 8g + 4hh .. +3 (element
    // e uses group e / 4); each group is read kLD steps before its first use
    constexpr int kLD = D == 64 ? 1 : 2;  // d = 64: keeps the kernel at 256 registers (2 waves per SIMD)
    f32x4 lg[8], dg[8];
    // step i: the reads of product i + kLA (and of the lse2 / D groups due),
    // then product i
    auto step_products = [&](auto I) __attribute__((always_inline)) {
      constexpr int i = decltype(I)::value;
      if constexpr (i + kLA < NPR) read(std::integral_constant<int, i + kLA>{});
      static_for<8>([&](auto G) __attribute__((always_inline)) {
        constexpr int g = decltype(G)::value;
        if constexpr (NS + 4 * g / EP - kLD == i)
          lg[g] = *reinterpret_cast<const f32x4*>(l2s + 8 * g + 4 * hh);
        if constexpr (2 * NS + 4 * g / ES - kLD == i)
          dg[g] = *reinterpret_cast<const f32x4*>(dds + 8 * g + 4 * hh);
      });
      product(I);
    };
    // element e of this lane's 32 (query, key) pairs is register 8(kc&1) + e%8
    // of half kc/2, kc = e/8; its row's lse2 / D are entry e%4 of group e/4
    auto pack = [&](const f32x16& x, int, auto KC) __attribute__((always_inline)) {
      constexpr int r0 = 8 * (decltype(KC)::value & 1);
      return to_bf16x8(x[r0], x[r0 + 1], x[r0 + 2], x[r0 + 3], x[r0 + 4], x[r0 + 5], x[r0 + 6], x[r0 + 7]);
    };

    static_for<kLA>(read);
    s[0] = s[1] = dp[0] = dp[1] = f32x16{};
    __builtin_amdgcn_sched_barrier(0);
    static_for<NS>([&](auto I) __attribute__((always_inline)) {
      step_products(I);
      __builtin_amdgcn_sched_barrier(0);
    });
    if constexpr (decltype(masked)::value) {
      // pair (query qi, key) visible iff qi < Sq, key < Skv and the causal /
      // window rule holds; as bounds on qi: vis_lo <= qi < vis_hi
      int64_t vis_lo = 0, vis_hi = Sq;
      if (p.causal) {
        vis_lo = max(int64_t(0), int64_t(key) - off);
        if (p.window > 0) vis_hi = min(int64_t(Sq), int64_t(key) - off + p.window);
      }
      if (!key_ok) vis_hi = 0;
      const int lo = int(max(min(vis_lo - i0, int64_t(kBQ)), int64_t(-1))) - 4 * hh;
      const int hi = int(max(min(vis_hi - i0, int64_t(kBQ)), int64_t(-1))) - 4 * hh;
#pragma unroll
      for (int qh = 0; qh < 2; ++qh) {
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const int qc0 = qh * 32 + 8 * (r >> 2) + (r & 3);
          if (qc0 < lo || qc0 >= hi) s[qh][r] = -INFINITY;
        }
      }
      __builtin_amdgcn_sched_barrier(0);
    }
    // dP steps, each with EP elements of P = 2^(s c - lse2)
    static_for<NS>([&](auto J) __attribute__((always_inline)) {
      constexpr int j = decltype(J)::value;
      step_products(std::integral_constant<int, NS + j>{});
      static_for<EP>([&](auto U) __attribute__((always_inline)) {
        constexpr int e = EP * j + decltype(U)::value;
        constexpr int kc = e / 8, qh = kc >> 1, r = 8 * (kc & 1) + e % 8;
        float x = s[qh][r];
        asm volatile("" : "+v"(x));
        float pe = __builtin_amdgcn_exp2f(fmaf(x, p.c, -lg[e / 4][e % 4]));
        asm volatile("" : "+v"(pe));
        s[qh][r] = pe;
      });
      if constexpr ((EP * (j + 1)) % 8 == 0) {
        constexpr int kc = EP * (j + 1) / 8 - 1;
        pf[kc] = pack(s[kc >> 1], 0, std::integral_constant<int, kc>{});
      }
      __builtin_amdgcn_sched_barrier(0);
    });
    // dV steps, each with ES elements of dS = P (dP - D)
    static_for<NT>([&](auto J) __attribute__((always_inline)) {
      constexpr int j = decltype(J)::value;
      step_products(std::integral_constant<int, 2 * NS + j>{});
      static_for<ES>([&](auto U) __attribute__((always_inline)) {
        constexpr int e = ES * j + decltype(U)::value;
        constexpr int kc = e / 8, qh = kc >> 1, r = 8 * (kc & 1) + e % 8;
        // element e % 8 of pf[kc] widened to fp32 from its packed dword
        const uint32_t pw = __builtin_bit_cast(u32x4, pf[kc])[(e % 8) / 2];
        float x = __builtin_bit_cast(float, (e & 1) ? (pw & 0xffff0000u) : (pw << 16)), y = dp[qh][r];
        asm volatile("" : "+v"(x), "+v"(y));
        float sv = x * (y - dg[e / 4][e % 4]);
        asm volatile("" : "+v"(sv));
        dp[qh][r] = sv;
      });
      if constexpr ((ES * (j + 1)) % 8 == 0) {
        constexpr int kc = ES * (j + 1) / 8 - 1;
        dsf[kc] = pack(dp[kc >> 1], 0, std::integral_constant<int, kc>{});
      }
      __builtin_amdgcn_sched_barrier(0);
    });
    // dK steps
    static_for<NT>([&](auto J) __attribute__((always_inline)) {
      step_products(std::integral_constant<int, 2 * NS + NT + decltype(J)::value>{});
      __builtin_amdgcn_sched_barrier(0);
    });
  };

  // Whether this wave's keys see any / every query of tile [i0, i0 + 64).
  auto tile_class = [&](int i0) __attribute__((always_inline)) {
    // returns 0: nothing visible, 1: some pairs masked, 2: all pairs visible
    if (jw >= Skv) return 0;
    const int qe = min(i0 + kBQ, Sq);  // one past the tile's last query
    if (p.causal) {
      if (int64_t(jw) > int64_t(qe) - 1 + off) return 0;  // every key after every diagonal
      if (p.window > 0 && int64_t(jwe) - 1 <= int64_t(i0) + off - p.window) return 0;
    }
    bool full = (i0 + kBQ <= Sq) && (jw + 32 <= Skv);
    if (p.causal) {
      full = full && int64_t(jwe) - 1 <= int64_t(i0) + off;
      if (p.window > 0) full = full && int64_t(jw) > int64_t(qe) - 1 + off - p.window;
    }
    return full ? 2 : 1;
  };

  // (head, query tile) of the tile in the current stage and of the next
  // load, advanced by counting (iteration it is head g0 + it / ntq, tile
  // tq0 + it % ntq)
  int cur_i0 = tq0 * kBQ, ld_g = g0, ld_tq = 0;
  auto advance = [&]() __attribute__((always_inline)) {
    if (++ld_tq == ntq) {
      ld_tq = 0;
      ++ld_g;
    }
  };
  auto step = [&](int it, char* cur, char* nxt) __attribute__((always_inline)) {
    wait_vmcnt<0>();
    __syncthreads();
    const int i0 = cur_i0;
    if (it + 1 < niter) {
      advance();
      cur_i0 = (tq0 + ld_tq) * kBQ;
      issue_loads(ld_g, cur_i0, nxt);
    }
    const int cls = tile_class(i0);
    if (cls == 2) {
      compute(i0, cur, std::false_type{});
    } else if (cls == 1) {
      compute(i0, cur, std::true_type{});
    }
  };
  if (niter > 0) issue_loads(g0, cur_i0, lds);
  for (int it = 0; it < niter; it += 2) {
    step(it, lds, lds + STAGE_B);
    if (it + 1 < niter) step(it + 1, lds + STAGE_B, lds);
  }

  // ---- dK = scale * (Q^T dS)^T, dV = (dO^T P)^T: bf16 (RNE), or fp32
  // partials of this head split
  if (p.nsplit > 1) {
    if (!key_ok) return;
    const int64_t ko = ((int64_t(b) * Skv + key) * p.Hkv + hk) * D;
    const int64_t po = int64_t(split) * p.B * Skv * p.Hkv * D + ko;
#pragma unroll
    for (int nb = 0; nb < NB; ++nb) {
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        f32x4 kv4, vv4;
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          kv4[e] = acck[nb][4 * g + e] * p.scale;
          vv4[e] = accv[nb][4 * g + e];
        }
        *reinterpret_cast<f32x4*>(p.part_k + po + nb * 32 + 8 * g + 4 * hh) = kv4;
        *reinterpret_cast<f32x4*>(p.part_v + po + nb * 32 + 8 * g + 4 * hh) = vv4;
      }
    }
    return;
  }
  // whole key rows through the stage the last step did not read (idle once
  // that step's barrier has passed; each wave uses its own quarter, first for
  // dK, then for dV)
  char* stage = lds + (niter & 1) * STAGE_B + w * 32 * ROWB;
  const int64_t kvrow0 = (int64_t(b) * Skv + jw) * p.Hkv + hk;  // this wave's first key row
  auto key_off = [&](int r) -> uint32_t {
    return jw + r < Skv ? uint32_t(r * p.Hkv) * uint32_t(2 * D) : kSkipRow;
  };
  store_tile_rows_bf16<D>(stage, acck, p.scale, reinterpret_cast<char*>(p.dk + kvrow0 * D), key_off);
  store_tile_rows_bf16<D>(stage, accv, 1.f, reinterpret_cast<char*>(p.dv + kvrow0 * D), key_off);
}

// Sums the head-split partials of dK and dV in split order -> bf16; 8
// elements per thread.
__global__ __launch_bounds__(256) void bwd_reduce_kernel(BwdParams p, int64_t n) {
  const int64_t e = (int64_t(blockIdx.x) * 256 + threadIdx.x) * 8;
  if (e >= n) return;
  f32x4 k0{}, k1{}, v0{}, v1{};
  for (int s = 0; s < p.nsplit; ++s) {
    const int64_t o = int64_t(s) * n + e;
    k0 += *reinterpret_cast<const f32x4*>(p.part_k + o);
    k1 += *reinterpret_cast<const f32x4*>(p.part_k + o + 4);
    v0 += *reinterpret_cast<const f32x4*>(p.part_v + o);
    v1 += *reinterpret_cast<const f32x4*>(p.part_v + o + 4);
  }
  *reinterpret_cast<bf16x8*>(p.dk + e) = to_bf16x8(k0[0], k0[1], k0[2], k0[3], k1[0], k1[1], k1[2], k1[3]);
  *reinterpret_cast<bf16x8*>(p.dv + e) = to_bf16x8(v0[0], v0[1], v0[2], v0[3], v1[0], v1[1], v1[2], v1[3]);
}

int heads_per_chunk_shift(int G) {
  int s = 0;
  while (s < 5 && (G % (2 << s)) == 0) ++s;  // largest power of two <= 32 dividing G
  return s;
}

template <int D>
hipError_t launch_all(const BwdParams& p, int64_t dq_blocks, int64_t kv_blocks, hipStream_t stream) {
  // each kernel reads what the previous ones wrote (the dQ kernel fills the
  // row statistics the dK/dV kernel reads): stop at the first launch that
  // fails, so none runs on a workspace that was never filled
  hipError_t err = launch_kernel(bwd_dq_kernel<D>, dim3(unsigned(dq_blocks)), dim3(kThreads), 0, stream, p);
  if (err == hipSuccess)
    err = launch_kernel(bwd_dkdv_kernel<D>, dim3(unsigned(kv_blocks)), dim3(kThreads), 0, stream, p);
  if (err == hipSuccess && p.nsplit > 1) {
    const int64_t n = int64_t(p.B) * p.Skv * p.Hkv * D;
    const int64_t blocks = (n / 8 + 255) / 256;
    err = launch_kernel(bwd_reduce_kernel, dim3(unsigned(blocks)), dim3(256), 0, stream, p, n);
  }
  return err;
}

}  // namespace

int bwd_head_splits(int B, int Hq, int Hkv, int Skv) {
  // enough (b, kv head, split, key block) blocks for about four per CU
  const int64_t G = Hq / Hkv;
  const int64_t blocks = int64_t(B) * Hkv * ((int64_t(Skv) + kBK - 1) / kBK);
  int64_t want = (1024 + blocks - 1) / blocks;
  if (want > G) want = G;
  if (want < 1) want = 1;
  const int64_t hps = (G + want - 1) / want;
  return int((G + hps - 1) / hps);
}

hipError_t launch_bwd_bf16(const BwdArgs& a, hipStream_t stream) {
  BwdParams p;
  p.q = static_cast<const __bf16*>(a.q);
  p.k = static_cast<const __bf16*>(a.k);
  p.v = static_cast<const __bf16*>(a.v);
  p.o = static_cast<const __bf16*>(a.o);
  p.dout = static_cast<const __bf16*>(a.dout);
  p.lse = a.lse;
  p.dq = static_cast<__bf16*>(a.dq);
  p.dk = static_cast<__bf16*>(a.dk);
  p.dv = static_cast<__bf16*>(a.dv);
  p.l2 = a.l2;
  p.dd = a.dd;
  p.B = a.B;
  p.Hq = a.Hq;
  p.Hkv = a.Hkv;
  p.Sq = a.Sq;
  p.Skv = a.Skv;
  p.G = a.Hq / a.Hkv;
  p.gc_shift = heads_per_chunk_shift(p.G);
  p.nchunk = p.G >> p.gc_shift;
  const int rows_pos = kBM >> p.gc_shift;
  p.nqb = (a.Sq + rows_pos - 1) / rows_pos;
  p.nx = a.B * a.Hkv * p.nchunk;
  const float c = std::fabs(a.scale) * kLog2e;
  p.c = c < 1e-30f ? 1e-30f : c;
  p.scale = a.scale;
  p.negate = a.scale < 0.f ? 1 : 0;
  p.causal = a.causal;
  p.window = a.window;
  p.nsplit = bwd_head_splits(a.B, a.Hq, a.Hkv, a.Skv);
  p.hps = (p.G + p.nsplit - 1) / p.nsplit;
  p.part_k = a.part_k;
  p.part_v = a.part_v;
  if (p.nsplit > 1 && (!p.part_k || !p.part_v)) return hipErrorInvalidValue;
  const int64_t dq_blocks = int64_t(p.nqb) * p.nx;
  const int64_t kv_blocks = int64_t(a.B) * a.Hkv * p.nsplit * ((a.Skv + kBK - 1) / kBK);
  if (dq_blocks > 0x7fffffff || kv_blocks > 0x7fffffff) return hipErrorInvalidConfiguration;
  p.div_nx = UDiv::make(uint32_t(p.nx));
  p.div_nchunk = UDiv::make(uint32_t(p.nchunk));
  p.div_hkv = UDiv::make(uint32_t(p.Hkv));
  p.div_nbh = UDiv::make(uint32_t(a.B * a.Hkv * p.nsplit));
  p.div_nsplit = UDiv::make(uint32_t(p.nsplit));
  if (a.d == 64) return launch_all<64>(p, dq_blocks, kv_blocks, stream);
  return launch_all<128>(p, dq_blocks, kv_blocks, stream);
}

}  // namespace fattn
