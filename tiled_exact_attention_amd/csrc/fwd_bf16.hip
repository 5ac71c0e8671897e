// bf16 tiled exact attention on the gfx950 matrix cores.
//
// Method ([FA-NPU] tiling section; [FA-3MOVES] moves 1 and 2): a block owns a
// tile of query rows and streams key/value tiles through LDS; per tile it
// forms the scores with matrix-core products, folds them into a running row
// max m and row sum l (rescaling the accumulator by 2^(m_old - m_new) when
// the max grows), and accumulates P.V.  Scores never leave registers.
//
// gfx950 design:
//  * 256 threads = 4 waves; each wave owns 32 query rows, the block 128.
//    Rows enumerate (position, query head) with the head fastest inside a
//    chunk of GC heads that share one kv head (GQA/MQA, [FA-VARIANTS] GQA
//    section): one K/V tile in LDS serves GC heads x 128/GC positions, and no
//    K/V copy is ever made.
//  * scores are computed transposed, S^T = K Q^T, with
//    v_mfma_f32_32x32x16_bf16 (A = K rows from LDS, B = the wave's Q rows
//    held in registers).  In that output layout each lane holds one query
//    row and 16 keys, so the probabilities are already the B operand of
//    O^T += V^T P^T, and the accumulator of each lane is its own query row:
//    the softmax row statistics need one cross-lane step (lane ^ 32).
//  * V^T is read from a row-major V tile with ds_read_b64_tr_b16, the
//    transposing LDS read, in the key order the P layout dictates.
//  * K/V tiles of 64 keys are filled straight from HBM into LDS by
//    buffer_load_dwordx4 ... lds (no register staging), two K and two V buffers.
//    Each wave is software-pipelined by one tile: iteration t multiplies
//    S(t) = K(t) Q^T and O += V(t-1)^T P(t-1) in one block of matrix
//    products, then turns S(t) into P(t).  The products of one iteration are
//    independent, so they are issued as interleaved chains with their LDS
//    operand reads running a few products ahead; the softmax of one wave
//    overlaps the products of the other wave on its SIMD.  K(t+1) and V(t)
//    stream in during iteration t.  LDS rows are XOR-swizzled in 16-byte
//    chunks so neither read pattern has bank conflicts; each lane's LDS read
//    offsets are computed once, the buffer and block offsets are immediates.
//  * causal/window: blocks visit only key tiles that intersect their visible
//    band; the mask is applied only on tiles that straddle a band edge (keys
//    a row cannot see get probability exactly 0).  Heavy (late) query blocks
//    are dispatched first.
//  * softmax in base 2 with the scale folded in: p = 2^(s*c - m), c =
//    scale*log2(e); a negative scale is applied as an exact sign flip of Q.
#include "device_util.h"
#include "launch.h"

#include <cmath>
#include <type_traits>

namespace fattn {
namespace {

constexpr int kWaves = 4;
constexpr int kThreads = 64 * kWaves;
constexpr int kBM = 32 * kWaves;  // query rows per block
constexpr int kBN = 64;           // keys per tile
constexpr float kNegHuge = -1e30f;
constexpr float kLn2 = 0.693147180559945309f;
// The accumulator and row sum are kept relative to a reference max m_ref
// (base-2 units), set to the row max on a wave's first tile and afterwards
// raised only when some probability of a tile would exceed 2^kLazy.  A lane's
// partial sum of the tile's probabilities exceeds 2^kLazy whenever one of
// them does, so the steady state tests that sum and takes no max over the
// scores; only then is the tile's max taken and its probabilities recomputed.
// Numerator and denominator share m_ref, so the result is the same softmax.
constexpr float kLazy = 8.f;
constexpr float kSumLimit = 256.f;  // 2^kLazy
// LDS operand reads are issued this many matrix products ahead of their use.
constexpr int kLA = 3;

// sched_group_barrier sequences: N instructions of class M (0x008 matrix
// product, 0x100 LDS read), or REP repetitions of (N1 of M1, N2 of M2).
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

struct Params {
  const __bf16* q;
  const __bf16* k;
  const __bf16* v;
  __bf16* o;
  float* lse;
  int Hq, Hkv, Sq, Skv;
  int G;         // query heads per kv head
  int gc_shift;  // log2 of the heads per row chunk (GC)
  int nchunk;    // G / GC
  int nqb;       // row blocks per (b, kv head, head chunk)
  int nx;        // B * Hkv * nchunk
  float c;       // |scale| * log2(e), >= 1e-30
  int negate;    // 1 if scale < 0 (Q sign flipped on load)
  int causal, window;
  // packed variable-length batch (null: the dense [B, S, H, d] layout)
  const int* cu_q;
  const int* cu_k;
  int total_q, total_k;
  UDiv div_nx, div_nqb, div_nchunk, div_hkv;  // by nx, nqb, nchunk and Hkv
};

template <int D>
__global__ __launch_bounds__(kThreads, 2) void fwd_bf16_kernel(Params p) {
  constexpr int KCH = D / 8;                 // 16-byte chunks per K/V row
  constexpr int ROWB = D * 2;                // bytes per K/V row
  constexpr int TILE_B = kBN * ROWB;         // bytes of one K (or V) tile
  constexpr int LPI = 1024 / ROWB;           // rows filled by one 1 KB LDS-DMA instruction
  constexpr int NLD = kBN / (kWaves * LPI);  // LDS-DMA instructions per wave per tensor per tile
  constexpr int KSTEPS = D / 16;             // k-steps of the QK^T product
  constexpr int NB = D / 32;                 // 32-wide blocks of the output row
  static_assert(NLD * LPI * kWaves == kBN, "tile rows must split evenly over the waves");
  static_assert(4 * TILE_B <= 65536, "LDS read offsets fit the 16-bit immediate");
  // LDS: two K buffers and two V buffers, one tile each (the K buffers also
  // stage the output rows in the epilogue)
  __shared__ __attribute__((aligned(1024))) char lds_k0[TILE_B];
  __shared__ __attribute__((aligned(1024))) char lds_k1[TILE_B];
  __shared__ __attribute__((aligned(1024))) char lds_v0[TILE_B];
  __shared__ __attribute__((aligned(1024))) char lds_v1[TILE_B];
  char* const kbuf[2] = {lds_k0, lds_k1};
  char* const vbuf[2] = {lds_v0, lds_v1};

  // ---- block -> (batch, kv head, head chunk, query block); heavy blocks first.
  // Workgroups go to the 8 XCDs round-robin (id % 8).  Dense batches number
  // blocks query-block-major over all (b, kv head, chunk) pairs: the heaviest
  // blocks of every pair go first, so the tail is light.  Packed
  // variable-length batches (with pairs a multiple of 8) instead give XCD j
  // the pairs j, j+8, ... one after another, heavy-first within each pair:
  // one XCD then works on one or two sequences at a time rather than on all of
  // them.  Measured on MI355X for 8 GQA sequences of 256..4096 tokens: 754 ->
  // 456 us; for dense batches it was no faster (MHA B=2: slower, a later
  // heavy tail per XCD).
  const int id = blockIdx.x;
  int x, slot;
  if (p.cu_q && (p.nx & 7) == 0) {
    const int xcd = id & 7, l = id >> 3;
    const int pair = int(p.div_nqb.div(uint32_t(l)));
    slot = l - pair * p.nqb;
    x = pair * 8 + xcd;
  } else {
    slot = int(p.div_nx.div(uint32_t(id)));
    x = id - slot * p.nx;
  }
  const int qb = p.causal ? p.nqb - 1 - slot : slot;
  const int xc = int(p.div_nchunk.div(uint32_t(x)));  // x / nchunk
  const int chunk = x - xc * p.nchunk;
  const int b = int(p.div_hkv.div(uint32_t(xc)));
  const int hk = xc - b * p.Hkv;
  const int gc = 1 << p.gc_shift;
  const int rows_pos = kBM >> p.gc_shift;     // positions per block
  const int p0 = qb * rows_pos;
  const int hq0 = hk * p.G + chunk * gc;
  const SeqView sv = seq_view(p.cu_q, p.cu_k, p.total_q, p.total_k, b, p.Hq, p.Sq, p.Skv);
  const int Sq = sv.Sq, Skv = sv.Skv;
  if (p0 >= Sq) return;  // a row block past this sequence's end (block-uniform)

  const int lane = threadIdx.x & 63;
  const int w = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);  // wave index (scalar)
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
  int row_lo = 0, row_hi = Skv;
  if (p.causal) {
    je = min(int64_t(Skv), bpos_hi + off + 1);
    row_hi = int(min(int64_t(Skv), pos + off + 1));
    if (p.window > 0) {
      jb = max(int64_t(0), p0 + off - p.window + 1);
      row_lo = int(max(int64_t(0), pos + off - p.window + 1));
    }
  }
  const int ntiles = je > jb ? int((je - jb + kBN - 1) / kBN) : 0;
  // the lowest row_hi and the highest row_lo among the wave's rows (its first
  // and last rows; wave-uniform)
  int w_lo_max = 0, w_hi_min = Skv;
  if (p.causal) {
    const int pos_a = p0 + ((w * 32) >> p.gc_shift), pos_b = p0 + ((w * 32 + 31) >> p.gc_shift);
    w_hi_min = int(min(int64_t(Skv), pos_a + off + 1));
    if (p.window > 0) w_lo_max = int(max(int64_t(0), pos_b + off - p.window + 1));
  }

  // ---- Q rows of this wave as the B operand (k-step m: columns 16m + 8hh .. +7)
  bf16x8 qf[KSTEPS];
  {
    const __bf16* qrow = p.q + ((sv.q_row0 + (row_ok ? pos : 0)) * p.Hq + hq) * D;
    const uint32_t sign = p.negate ? 0x80008000u : 0u;  // uniform: one xor per dword
#pragma unroll
    for (int m = 0; m < KSTEPS; ++m) {
      uint4 raw = *reinterpret_cast<const uint4*>(qrow + 16 * m + 8 * hh);
      raw.x ^= sign; raw.y ^= sign; raw.z ^= sign; raw.w ^= sign;
      qf[m] = __builtin_bit_cast(bf16x8, raw);
    }
  }

  // ---- LDS layout: row r of a tile at r*ROWB, its 16-byte chunk c stored at
  // position c ^ swz(r).  Per-lane byte offsets, fixed for the whole kernel:
  //  K reads (A operand of S^T = K Q^T): row lq (+32 for the second key block),
  //  chunk 2m + hh;  V reads (transposed, A operand of O^T = V^T P^T): rows
  //  16kc + 4*h2 + (s16 >> 2) + 8R, columns nb*32 + 16*nh + 4*(s16 & 3).
  int koff[KSTEPS];
#pragma unroll
  for (int m = 0; m < KSTEPS; ++m) koff[m] = lq * ROWB + (((2 * m + hh) ^ swz<D>(lq)) << 4);
  const int g16 = lane >> 4, s16 = lane & 15;
  const int h2 = g16 >> 1, nh = g16 & 1;
  int voff[NB][2];
#pragma unroll
  for (int nb = 0; nb < NB; ++nb) {
#pragma unroll
    for (int R = 0; R < 2; ++R) {
      const int r = 4 * h2 + (s16 >> 2) + 8 * R;
      const int col = nb * 32 + nh * 16 + 4 * (s16 & 3);
      voff[nb][R] = r * ROWB + (((col >> 3) ^ swz<D>(r)) << 4) + (col & 7) * 2;
    }
  }

  // ---- LDS-DMA load assignment: wave w fills rows 16w .. 16w+15 of a tile;
  // instruction i covers rows 16w + LPI*i + (lane / KCH), lane's physical
  // chunk lane % KCH holds logical chunk (lane % KCH) ^ swz(row).
  const int64_t kv_stride = int64_t(p.Hkv) * D;
  const __bf16* kbase = p.k + (sv.k_row0 * p.Hkv + hk) * D;
  const __bf16* vbase = p.v + (sv.k_row0 * p.Hkv + hk) * D;
  // byte offset of this lane's source chunk from the first row of a tile
  // (non-negative and below 2^31: 64 rows of Hkv * d elements, checked on
  // the host), so every copy addresses a scalar base plus a 32-bit lane
  // offset and no lane holds a 64-bit address (measured on MI355X: 28 fewer
  // registers at d = 128, bit-identical, 1-2% faster at d = 128)
  uint32_t goff[NLD];
  const int lr = lane / KCH;
  const uint32_t row_b = uint32_t(kv_stride) * 2u;  // bytes per key row
#pragma unroll
  for (int i = 0; i < NLD; ++i) {
    const int r = 16 * w + LPI * i + lr;
    goff[i] = uint32_t(r) * row_b + uint32_t(((lane % KCH) ^ swz<D>(r)) * 16);
  }
  // copy rows j0 .. j0+63 of one tensor (K or V) into an LDS buffer; on the
  // last tile of the sequence, rows past the end re-read the last row
  auto issue_tile = [&](const __bf16* base, int64_t j0, char* dst_tile) __attribute__((always_inline)) {
    const char* src = reinterpret_cast<const char*>(base + j0 * kv_stride);
    if (int(j0) + kBN <= Skv) {  // j0 < Skv < 2^31: a scalar compare
#pragma unroll
      for (int i = 0; i < NLD; ++i)
        buffer_to_lds16(src, goff[i], dst_tile + (16 * w + LPI * i) * ROWB);
    } else {
      const int last = int(Skv - 1 - j0);  // last row of the sequence within this tile
#pragma unroll
      for (int i = 0; i < NLD; ++i) {
        const int r = 16 * w + LPI * i + lr;
        const uint32_t back = uint32_t(max(r - last, 0)) * row_b;
        buffer_to_lds16(src, goff[i] - back, dst_tile + (16 * w + LPI * i) * ROWB);
      }
    }
  };

  f32x16 acc[NB];
#pragma unroll
  for (int nb = 0; nb < NB; ++nb) acc[nb] = f32x16{};
  float m_run = kNegHuge, l_run = 0.f;

  f32x16 s[2];   // S^T of the current tile (two 32-key blocks)
  bf16x8 pf[4];  // P of the previous tile, the B operand of O^T += V^T P^T

  // ---- one block of matrix products: S(t) = K(t) Q^T over the first QK
  // 32-key blocks of the tile, and O^T += V(t-1)^T P(t-1)^T over the first PV
  // 32-key blocks of the previous tile (QK, PV in 0..2).  The products are
  // issued as interleaved accumulation chains; the LDS operand reads are
  // placed kLA products ahead of their use (sched_group_barrier: 0x100 = LDS
  // read, 0x008 = matrix product).
  auto products = [&](const char* kt, const char* vt, auto QK, auto PV) __attribute__((always_inline)) {
    constexpr int qk = decltype(QK)::value, pv = decltype(PV)::value;
    constexpr int NQK = qk * KSTEPS, NPV = 2 * pv * NB;  // products; K reads = NQK, V^T reads = 2 * NPV
    // A distinct marker per variant keeps the compiler from hoisting the
    // operand reads the variants share above the branch that selects them
    // (which would hold all of them in registers at once).
    if constexpr (qk == 2 && pv == 2) {
      asm volatile("; products: S and PV" ::: "memory");
    } else if constexpr (qk == 1 && pv == 2) {
      asm volatile("; products: S (first half) and PV" ::: "memory");
    } else if constexpr (qk == 2) {
      asm volatile("; products: S" ::: "memory");
    } else if constexpr (pv == 2) {
      asm volatile("; products: PV" ::: "memory");
    } else {
      asm volatile("; products: PV (first half)" ::: "memory");
    }
    if constexpr (qk > 0) {
      bf16x8 ka[KSTEPS][2];
#pragma unroll
      for (int m = 0; m < KSTEPS; ++m)
#pragma unroll
        for (int kb = 0; kb < qk; ++kb) ka[m][kb] = *reinterpret_cast<const bf16x8*>(kt + koff[m] + kb * 32 * ROWB);
#pragma unroll
      for (int kb = 0; kb < qk; ++kb) s[kb] = f32x16{};
#pragma unroll
      for (int m = 0; m < KSTEPS; ++m)
#pragma unroll
        for (int kb = 0; kb < qk; ++kb) s[kb] = mfma32(ka[m][kb], qf[m], s[kb]);
    }
    if constexpr (pv > 0) {
#pragma unroll
      for (int kc = 0; kc < 2 * pv; ++kc) {
#pragma unroll
        for (int nb = 0; nb < NB; ++nb) {
          const i16x4 a0 = lds_read_tr16(vt + voff[nb][0] + kc * 16 * ROWB);
          const i16x4 a1 = lds_read_tr16(vt + voff[nb][1] + kc * 16 * ROWB);
          acc[nb] = mfma32(__builtin_bit_cast(bf16x8, concat_i16x4(a0, a1)), pf[kc], acc[nb]);
        }
      }
    }
    if constexpr (qk > 0 && pv > 0) {
      sched_group<0x100, 2 * kLA>();
      sched_pairs<0x008, 1, 0x100, 1, NQK>();
      sched_pairs<0x008, 1, 0x100, 2, NPV - kLA>();
      sched_group<0x008, kLA>();
    } else if constexpr (qk > 0) {
      sched_group<0x100, 2 * kLA>();
      sched_pairs<0x008, 1, 0x100, 1, NQK - 2 * kLA>();
      sched_group<0x008, 2 * kLA>();
    } else if constexpr (pv > 0) {
      sched_group<0x100, 2 * kLA>();
      sched_pairs<0x008, 1, 0x100, 2, NPV - kLA>();
      sched_group<0x008, kLA>();
    }
  };
  using None = std::integral_constant<int, 0>;
  using Half = std::integral_constant<int, 1>;
  using Full = std::integral_constant<int, 2>;

  // ---- S(t) -> P(t): mask (only on tiles that may straddle an edge of the
  // block's band), online softmax in base 2 with the scale folded into c.
  auto softmax = [&](int64_t j0, auto masked, auto first, auto NKB) __attribute__((always_inline)) {
    constexpr int nkb = decltype(NKB)::value;  // 32-key blocks of S formed (the rest lie past the band)
    // key j0 + kofs is visible iff row_lo <= key < row_hi; kofs - 4*hh is a
    // compile-time constant per register, so compare against shifted bounds.
    // The bounds rise with the lane's row, so the wave's first and last rows
    // bound them all: scalar tests find the 32-key blocks of S that an edge
    // cuts for some row of the wave, and only those get per-element compares
    // (one per element and edge).
    if constexpr (decltype(masked)::value) {
      const int jj = int(j0);  // j0 < Skv fits an int
      // each test guards a plain if-then that updates s in place (no else
      // branch), so the results stay in the registers of s
#pragma unroll
      for (int kb = 0; kb < nkb; ++kb) {
        const int b0 = jj + 32 * kb;  // first key of the block
        if (w_hi_min < b0 + 32) {     // the causal edge (or the end of the keys) cuts the block for some row
          const int hi = row_hi - b0 - 4 * hh;
#pragma unroll
          for (int r = 0; r < 16; ++r) {
            const int kc0 = 8 * (r >> 2) + (r & 3);
            if (kc0 >= hi) s[kb][r] = -INFINITY;
          }
        }
        if (w_lo_max > b0) {  // the window edge cuts the block for some row
          const int lo = row_lo - b0 - 4 * hh;
#pragma unroll
          for (int r = 0; r < 16; ++r) {
            const int kc0 = 8 * (r >> 2) + (r & 3);
            if (kc0 < lo) s[kb][r] = -INFINITY;
          }
        }
      }
    }
    auto raise_reference = [&]() __attribute__((always_inline)) {
      float mx = kNegHuge;
#pragma unroll
      for (int kb = 0; kb < nkb; ++kb) {
#pragma unroll
        for (int r = 0; r < 16; ++r) mx = fmaxf(mx, s[kb][r]);
      }
      mx = max_across_halves(mx) * p.c;
      return mx;
    };
    auto rescale_to = [&](float m_new) __attribute__((always_inline)) {
      const float alpha = __builtin_amdgcn_exp2f(m_run - m_new);
      m_run = m_new;
      l_run *= alpha;
#pragma unroll
      for (int nb = 0; nb < NB; ++nb) acc[nb] *= alpha;
    };
    auto exponentials = [&]() __attribute__((always_inline)) {
      float ps = 0.f;
#pragma unroll
      for (int kc = 0; kc < 2 * nkb; ++kc) {
        float e[8];
#pragma unroll
        for (int i = 0; i < 8; ++i) {
          e[i] = __builtin_amdgcn_exp2f(fmaf(s[kc >> 1][8 * (kc & 1) + i], p.c, -m_run));
          ps += e[i];
        }
        pf[kc] = to_bf16x8(e[0], e[1], e[2], e[3], e[4], e[5], e[6], e[7]);
      }
      return ps;
    };
    if constexpr (decltype(first)::value) {
      // first tile of the wave: the reference is the row max (the accumulator
      // and the row sum are still zero, so nothing is rescaled)
      m_run = fmaxf(m_run, raise_reference());
      l_run += exponentials();
    } else {
      // later tiles keep the reference unless some exponential exceeds 2^kLazy,
      // which the lane's partial sum reveals without a max over the scores
      float ps = exponentials();
      if (__builtin_expect(__any(ps > kSumLimit), 0)) {  // rare: raise the reference
        const float mx = raise_reference();
        rescale_to(fmaxf(m_run, mx));
        ps = exponentials();
      }
      l_run += ps;
    }
  };

  // ---- main loop.  Iteration t (0 <= t <= ntiles): K(t) and V(t-1) are in
  // LDS (K buffer t % 2, V buffer (t-1) % 2); K(t+1) and V(t) are copied
  // into the other buffers meanwhile.  Every buffer a copy overwrites was
  // last read in iteration t-1, which all waves have left at the barrier.
  // Iteration 0 forms S(0) only, iteration ntiles only adds V(ntiles-1)^T
  // P(ntiles-1)^T; every other one does both, so the steady state has no
  // branches.  Every wave takes every tile of the block's band: keys a row
  // cannot see get probability exactly 0.  Tiles [t_lo, t_hi) are fully
  // visible to every row of the block and skip the mask; the tiles before
  // t_lo (window edge) and from t_hi on (causal edge, end of the keys) are
  // masked, and so is tile 0 unless every row sees all of it.  Iterations
  // run in pairs (odd t, then even t) so the buffer offsets are
  // compile-time constants.
  // The copies are issued in buffer form (buffer_load ... lds): for the flat
  // form the compiler cannot prove that the operand reads miss the copies'
  // destinations (it waits for the copies, vmcnt(0), before the first V^T
  // read) and stops counting LDS reads precisely (every wait becomes
  // lgkmcnt(0)); the buffer form keeps both waits exact.  The copies of
  // iteration t go out after its products, so that the products start at
  // once and the copies overlap the softmax and the barrier; measured on
  // MI355X that order is the faster one for every head layout.
  auto begin = [&](int t) __attribute__((always_inline)) {
    wait_vmcnt<0>();   // this wave's copies of K(t) and V(t-1) have landed
    __syncthreads();   // ... and everyone's; everyone has left iteration t-1
    return jb + int64_t(t) * kBN;
  };
  auto copies = [&](int t, int64_t j0, char* knxt, char* vcur) __attribute__((always_inline)) {
    if (t + 1 < ntiles) issue_tile(kbase, j0 + kBN, knxt);
    if (t < ntiles) issue_tile(vbase, j0, vcur);
  };
  auto iteration = [&](int t, auto odd, auto masked) __attribute__((always_inline)) {
    constexpr int cur = decltype(odd)::value ? 1 : 0;
    const int64_t j0 = begin(t);
    products(kbuf[cur], vbuf[cur ^ 1], Full{}, Full{});
    copies(t, j0, kbuf[cur ^ 1], vbuf[cur]);
    softmax(j0, masked, std::false_type{}, Full{});
  };
  // The last tile of the band may hold keys of the band in its first 32 rows
  // only (a window band of W + 15 keys, say); then S is formed, and turned
  // into probabilities, for those 32 keys alone, and its P^T product skips
  // the second half.  The pair loops stop one tile early for it.
  const bool last_half = ntiles >= 2 && je - jb - int64_t(ntiles - 1) * kBN <= kBN / 2;
  const int nloop = last_half ? ntiles - 1 : ntiles;  // iterations of the pair loops
  auto pair = [&](int t, auto masked) __attribute__((always_inline)) {
    iteration(t, std::true_type{}, masked);
    if (t + 1 < nloop) iteration(t + 1, std::false_type{}, masked);
  };
  if (ntiles > 0) {
    int t_lo, t_hi;  // odd, t_lo <= t_hi, t_hi - t_lo even
    bool first_full;  // tile 0 fully visible to every row (no mask)
    {
      const int64_t hi_min = p.causal ? min(int64_t(Skv), p0 + off + 1) : int64_t(Skv);
      const int64_t lo_max = (p.causal && p.window > 0) ? max(int64_t(0), bpos_hi + off - p.window + 1) : 0;
      const int raw_hi = hi_min - jb >= kBN ? int(min(int64_t(ntiles), (hi_min - jb) / kBN)) : 0;
      const int raw_lo = lo_max > jb ? int(min(int64_t(raw_hi), (lo_max - jb + kBN - 1) / kBN)) : 0;
      first_full = raw_lo == 0 && raw_hi >= 1;
      t_lo = max(raw_lo, 1) | 1;
      t_hi = raw_hi > t_lo ? t_lo + ((raw_hi - t_lo) & ~1) : t_lo;
    }
    issue_tile(kbase, jb, lds_k0);
    {
      const int64_t j0 = begin(0);
      products(lds_k0, lds_v0, Full{}, None{});
      copies(0, j0, lds_k1, lds_v0);
      if (first_full) {
        softmax(j0, std::false_type{}, std::true_type{}, Full{});
      } else {
        softmax(j0, std::true_type{}, std::true_type{}, Full{});
      }
    }
    int t = 1;
    for (; t < t_lo && t < nloop; t += 2) pair(t, std::true_type{});
    for (; t < t_hi; t += 2) pair(t, std::false_type{});
    for (; t < nloop; t += 2) pair(t, std::true_type{});
    const int tl = ntiles - 1;  // K(tl) sits in K buffer tl % 2; V(tl) goes to V buffer tl % 2
    if (last_half) {
      // the last tile (never fully visible: its second half lies past the band)
      const int64_t j0 = begin(tl);
      products((tl & 1) ? lds_k1 : lds_k0, (tl & 1) ? lds_v0 : lds_v1, Half{}, Full{});
      copies(tl, j0, lds_k0, (tl & 1) ? lds_v1 : lds_v0);
      softmax(j0, std::true_type{}, std::false_type{}, Half{});
    }
    // last product: V(tl) sits in V buffer tl % 2
    begin(ntiles);
    if (last_half) {
      products(lds_k0, (tl & 1) ? lds_v1 : lds_v0, None{}, Half{});
    } else {
      products(lds_k0, (tl & 1) ? lds_v1 : lds_v0, None{}, Full{});
    }
  }

  // ---- epilogue: normalise, write O (bf16, RNE) and lse (natural log).
  // Each wave stages its 32 output rows in its own quarter of the two K
  // buffers, which no wave reads and no copy targets after the barrier that
  // opened the last iteration, and writes whole rows with 16-byte stores.
  // Measured on MI355X: 2-5% off the launch (the epilogue of a 128-row block
  // went from about 2.7 to 1.8 us).
  const float l_tot = l_run + __shfl_xor(l_run, 32);
  const float inv = l_tot > 0.f ? 1.f / l_tot : 0.f;
  // rows of the block start at (position p0, head hq0); a row's byte offset
  // from there is below 2^32 (128 positions of Hq * d elements, checked on
  // the host)
  char* obase = reinterpret_cast<char*>(p.o + ((sv.q_row0 + p0) * p.Hq + hq0) * D);
  const int so = w * 32 * ROWB;  // this wave's staging rows: K buffer 0, then K buffer 1
  store_tile_rows_bf16<D>(so < TILE_B ? lds_k0 + so : lds_k1 + (so - TILE_B), acc, inv, obase,
                          [&](int r) -> uint32_t {
    const int prow = w * 32 + r;
    const int dpos = prow >> p.gc_shift;
    return p0 + dpos < Sq ? uint32_t(dpos * p.Hq + (prow & (gc - 1))) * uint32_t(2 * D) : kSkipRow;
  });
  if (!row_ok) return;
  if (hh == 0 && p.lse) {
    p.lse[sv.lse0 + int64_t(hq) * sv.lse_hs + pos] =
        l_tot > 0.f ? m_run * kLn2 + logf(l_tot) : -INFINITY;
  }
}

int heads_per_chunk_shift(int G) {
  int s = 0;
  while (s < 5 && (G % (2 << s)) == 0) ++s;  // largest power of two <= 32 dividing G
  return s;
}

}  // namespace

hipError_t launch_fwd_bf16(const FwdArgs& a, hipStream_t stream) {
  Params p;
  p.q = static_cast<const __bf16*>(a.q);
  p.k = static_cast<const __bf16*>(a.k);
  p.v = static_cast<const __bf16*>(a.v);
  p.o = static_cast<__bf16*>(a.o);
  p.lse = a.lse;
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
  float c = std::fabs(a.scale) * 1.4426950408889634f;
  p.c = c < 1e-30f ? 1e-30f : c;
  p.negate = a.scale < 0.f ? 1 : 0;
  p.causal = a.causal;
  p.window = a.window;
  p.cu_q = a.cu_q;
  p.cu_k = a.cu_k;
  p.total_q = a.total_q;
  p.total_k = a.total_k;
  const int64_t blocks = int64_t(p.nqb) * p.nx;
  if (blocks > 0x7fffffff) return hipErrorInvalidConfiguration;
  p.div_nx = UDiv::make(uint32_t(p.nx));
  p.div_nqb = UDiv::make(uint32_t(p.nqb));
  p.div_nchunk = UDiv::make(uint32_t(p.nchunk));
  p.div_hkv = UDiv::make(uint32_t(p.Hkv));
  return launch_kernel(a.d == 64 ? fwd_bf16_kernel<64> : fwd_bf16_kernel<128>,
                       dim3(unsigned(blocks)), dim3(kThreads), 0, stream, p);
}

}  // namespace fattn
