// Split-KV decode over an int8 or int4 KV cache, then a log-sum-exp merge.
//
// Method: one query token per sequence attends to all cached tokens.  The
// cache keeps int8 codes (or int4 codes, two per byte, element 2i in the low
// nibble of byte i) with an fp32 scale per (token, kv head) and is used
// without a decompressed copy ([FA-3MOVES] move 3): codes are converted to
// bf16 in registers (exact) and the scales are applied to the scores (k
// scale) and to the probabilities (v scale).  The keys of each
// (batch, kv head) stream are cut into splits; each split runs the online
// softmax of the [FA-NPU] tiling section over its tokens and writes a
// normalised partial output and its log-sum-exp, and the partials are merged
// by log-sum-exp (global max of the partial lse, weights e^(lse_s - max)).
// Where a stream has at most kWgMaxSplits splits, its splits are the waves of
// one workgroup, which merges them in LDS after a barrier and writes the
// output: one launch, no partials in memory.  More splits than that write
// partials to the workspace and a second kernel merges them.  With a single
// split the split kernel writes the output and lse itself.  All three forms
// do the same arithmetic in the same order, so they give the same bits.
//
// gfx950 design (split kernel): one wave per (batch, kv head, chunk of <= 16
// query heads, split).  Per 32-token tile:
//  * K codes are loaded straight from HBM into the A-operand layout of
//    v_mfma_f32_16x16x32_bf16 (lane = token, 16 contiguous bytes = 16 head
//    dims), converted to bf16 and multiplied with the query heads (B operand,
//    kept in registers): S = K q^T, a 16-token x 16-head block per product.
//    The C layout puts one query head per lane and 4 tokens per register
//    group, which is the B-operand layout P^T needs for the value product.
//  * V codes are loaded coalesced (a row of 128 bytes per 8 lanes), staged in
//    a per-wave LDS tile (rows padded to 144 bytes so the 16-byte row pieces
//    of 16 rows cover all banks) and read back transposed with
//    ds_read_b64_tr_b8 in exactly the token order of the P^T registers; the
//    codes become the A operand of O^T += V^T P^T.
//  * loads run three tiles ahead of use through a four-slot register ring
//    (about 25 KB in flight per wave with int8 codes), which is what keeps
//    HBM busy: the kernel is bound by bytes in flight, not by arithmetic.
//    A call over the whole cache reads it once, so its loads of codes and
//    scales carry the non-temporal hint and stream past the caches (measured
//    on MI355X right after a prefill launch: 392 -> 345 us per call); calls
//    with per-sequence lengths keep plain loads (NT = false), see
//    load_stream16.
//    Scales arrive as one dword per lane per tile and are redistributed
//    through LDS.
//  * int4 codes: code + 8 (0 .. 15) placed in the low byte under a 0x43 high
//    byte is the bf16 bit pattern of 136 + code, exact, built with one byte
//    permute per two values.  The products then carry a bias: for the scores
//    it is 136 * sum(q) per query head, computed once with the same products
//    and subtracted; for the output it is 136 * sum(p') over the tokens,
//    accumulated by one more product per tile against a constant 136 operand
//    with the same bf16 probabilities, and subtracted at the end.  For K each
//    lane group holds d/4 contiguous dims of its token; a k-step takes one
//    dword (8 dims) in the order even dims, then odd dims, and the query
//    operand is permuted the same way.  For V one transposed read yields both
//    nibbles of a byte column: the low nibbles (even dims) and the high
//    nibbles (odd dims) feed two products.
#include "device_util.h"
#include "launch.h"

#include <cmath>
#include <mutex>

namespace fattn {
namespace {

constexpr int kTile = 32;                 // tokens per step of the split kernel
constexpr float kNegHuge = -1e30f;
constexpr float kLn2 = 0.693147180559945309f;
constexpr int kHeadsPerWave = 16;         // N of the 16x16x32 product
// The accumulator and row sum are kept relative to a reference max that is
// only raised when the running max exceeds it by more than kLazy (base-2
// units); the shared reference cancels in the normalisation.
constexpr float kLazy = 8.f;         // N of the 16x16x32 product

static_assert(kDecodeTile % kTile == 0, "split chunks must hold whole tiles");

// Most splits one workgroup can hold: one wave per split at two waves per
// SIMD (the split kernel's register budget) on the four SIMDs of a CU.
constexpr int kWgMaxSplits = kDecodeWgMaxSplits;
static_assert(kWgMaxSplits * 64 <= 1024, "a workgroup holds at most 16 waves");

struct SplitParams {
  const __bf16* q;
  const uint8_t* kq;
  const float* ks;
  const uint8_t* vq;
  const float* vs;
  float* part_o;
  float* part_lse;
  __bf16* o;    // final output [B, Hq, d] when nsplit == 1 (no merge)
  float* lse;   // final lse [B, Hq] or null, when nsplit == 1
  const int* seqlens;  // [B] tokens each sequence sees (first seqlens[b]), or null: all Skv
  int Hq, Hkv, Skv;
  int G;        // query heads per kv head
  int nhc;      // head chunks per kv head: ceil(G / 16)
  int nsplit;
  int chunk;    // tokens per split
  float c;      // scale * log2(e)
};

// Byte counts of one tile for a code width.
template <int D, int BITS>
struct Geom {
  static constexpr int RB = D * BITS / 8;         // bytes per token row
  static constexpr int KB = RB / 4;               // K bytes per lane per token (a quarter row)
  static constexpr int KW = KB / 4;               // ... in dwords
  static constexpr int CPR = RB / 16;             // 16-byte pieces per V row
  static constexpr int RPL = 64 / CPR;            // V rows per load instruction
  static constexpr int VLOADS = kTile / RPL;      // 16-byte V loads per lane per tile
  static constexpr int VSTRIDE = RB + 16;         // padded LDS row (bytes)
  static constexpr int NREAD = RB / 16;           // transposed V reads per tile
  // LDS of one wave: the staged V tile, then the tile's k and v scales
  static constexpr int WAVE_LDS = kTile * VSTRIDE + 2 * kTile * 4;
  // merge area of the workgroup form: partial outputs [split][head][D + 4]
  // (rows padded by 16 bytes so the 16 heads of a 16-byte store hit
  // different banks), then partial lse [split][head]
  static constexpr int MROW = D + 4;
};

// Dynamic LDS bytes of a split-kernel block of nw waves (nw > 1: the
// workgroup form, whose merge area reuses the waves' staging areas).
template <int D, int BITS>
constexpr size_t split_lds_bytes(int nw, int heads) {
  using GM = Geom<D, BITS>;
  const size_t stage = size_t(nw) * GM::WAVE_LDS;
  if (nw == 1) return stage;
  const size_t merge = size_t(nw) * heads * (GM::MROW + 1) * 4;
  return stage > merge ? stage : merge;
}

// bf16 of (136 + code) for 8 int4 codes: element e of lo4 / hi4 is the code
// in the low nibble of byte e (already 0 .. 15 = code + 8).  The two results'
// slot order is: bytes 0, 1 of the first source, bytes 2, 3, then the second.
constexpr uint32_t kBf16Hi128 = 0x43434343u;  // high byte of bf16 128 .. 255
__device__ __forceinline__ bf16x8 biased_bf16x8(uint32_t a4, uint32_t b4) {
  uint4 r;
  r.x = __builtin_amdgcn_perm(kBf16Hi128, a4, 0x04010400u);  // [a.b0, 0x43, a.b1, 0x43]
  r.y = __builtin_amdgcn_perm(kBf16Hi128, a4, 0x04030402u);  // [a.b2, 0x43, a.b3, 0x43]
  r.z = __builtin_amdgcn_perm(kBf16Hi128, b4, 0x04010400u);
  r.w = __builtin_amdgcn_perm(kBf16Hi128, b4, 0x04030402u);
  return __builtin_bit_cast(bf16x8, r);
}

// Loads of the cache stream: with NT the non-temporal hint (a call reading
// the whole cache once streams past the caches: 386 -> 339 us for the int8
// workload, 213 -> 191 us int4, interleaved medians on MI355X), without it
// plain loads (calls with per-sequence lengths, whose time is set by the few
// longest sequences streaming alone at the end: 283 -> 264 us with plain loads).
template <bool NT>
__device__ __forceinline__ uint4 load_stream16(const void* p) {
  if constexpr (NT) return load_nt16(p);
  else return *reinterpret_cast<const uint4*>(p);
}
template <bool NT>
__device__ __forceinline__ float load_stream4(const float* p) {
  if constexpr (NT) return __builtin_nontemporal_load(p);
  else return *p;
}

// KB bytes at src as dwords w[0 .. KB/4).
template <int KB, bool NT>
__device__ __forceinline__ void load_k(const uint8_t* src, uint32_t* w) {
  if constexpr (KB % 16 == 0) {
#pragma unroll
    for (int i = 0; i < KB / 16; ++i) {
      const uint4 x = load_stream16<NT>(src + 16 * i);
      w[4 * i] = x.x; w[4 * i + 1] = x.y; w[4 * i + 2] = x.z; w[4 * i + 3] = x.w;
    }
  } else {
    static_assert(KB == 8, "a quarter row is 8, 16 or 32 bytes");
    typedef unsigned u32x2 __attribute__((ext_vector_type(2)));
    u32x2 x;
    if constexpr (NT) x = __builtin_nontemporal_load(reinterpret_cast<const u32x2*>(src));
    else x = *reinterpret_cast<const u32x2*>(src);
    w[0] = x[0]; w[1] = x[1];
  }
}

// Register-ring depth: tiles in flight = slots - 1.  An int8 slot takes 33
// VGPRs (a fifth slot spills), an int4 slot 17; measured on MI355X with one
// wave per SIMD, 6 or 8 int4 slots were no faster than 4.
constexpr int kRingSlots = 4;

// Loads of one 32-token tile held in registers between issue and use.
template <int D, int BITS>
struct TileRegs {
  // K codes in the MFMA A layout: token 16*blk + l%16, a quarter row per lane
  // group (int8: 16-byte pieces g + 4u; int4: contiguous bytes KB*g ..)
  uint32_t k[2][Geom<D, BITS>::KW];
  uint4 v[Geom<D, BITS>::VLOADS];  // V codes, coalesced: 64 lanes x 16 bytes per load
  float sc;  // lane l < 32: k scale of token l; lane l >= 32: v scale of token l - 32
};

// WG = false: one wave per block, block id = ((b * Hkv + hk) * nhc + hc) *
// nsplit + split.  WG = true: one block per (b, hk, hc) with one wave per
// split (nsplit <= kWgMaxSplits waves), merged in LDS.
template <int D, int BITS, bool WG, bool NT>
__global__ __launch_bounds__(WG ? 64 * kWgMaxSplits : 64, 2) void decode_split_kernel(SplitParams p) {
  using GM = Geom<D, BITS>;
  constexpr int RB = GM::RB;
  constexpr int KB = GM::KB;
  constexpr int KM = D / 32;              // k-steps of the QK product (8 dims per lane each)
  constexpr int VLOADS = GM::VLOADS;
  constexpr int CPR = GM::CPR;
  constexpr int RPL = GM::RPL;
  constexpr int VSTRIDE = GM::VSTRIDE;
  constexpr int CB = D / 16;              // 16-dim blocks of the output (= products per tile)
  extern __shared__ __attribute__((aligned(16))) char dyn_lds[];
  const int wave = WG ? int(threadIdx.x >> 6) : 0;
  char* const vlds = dyn_lds + wave * GM::WAVE_LDS;                         // staged V codes
  float* const slds = reinterpret_cast<float*>(vlds + kTile * VSTRIDE);  // k scales, then v scales

  const int lane = threadIdx.x & 63;
  const int n = lane & 15;   // head slot (B/C column), also token row of A
  const int g = lane >> 4;   // lane group

  int id = blockIdx.x;
  int split;
  if constexpr (WG) {
    split = wave;
  } else {
    split = id % p.nsplit;
    id /= p.nsplit;
  }
  const int hc = id % p.nhc; id /= p.nhc;
  const int hk = id % p.Hkv;
  const int b = id / p.Hkv;
  const int head0 = hc * kHeadsPerWave;
  const int nheads = min(kHeadsPerWave, p.G - head0);
  const int hq = hk * p.G + head0 + n;      // this lane's query head (if n < nheads)
  const bool head_ok = n < nheads;

  const int64_t stream = int64_t(b) * p.Hkv + hk;
  const uint8_t* kbase = p.kq + stream * p.Skv * RB;
  const uint8_t* vbase = p.vq + stream * p.Skv * RB;
  const float* ksb = p.ks + stream * p.Skv;
  const float* vsb = p.vs + stream * p.Skv;

  // Variable lengths (clamped to [0, Skv]): each sequence's tokens are cut
  // into nsplit splits of ceil(len / nsplit) tokens rounded up to whole
  // tiles, so a batch shorter than the cache still uses every split slot
  // (with the capacity's chunk a sequence of Skv/4 tokens would use a
  // quarter of them).  Splits past the end are empty (o = 0, lse = -inf,
  // weight 0 in the merge).
  int len = p.Skv, chunk = p.chunk;
  if (p.seqlens) {
    len = min(max(p.seqlens[b], 0), p.Skv);
    chunk = max(kDecodeTile, ((len + p.nsplit - 1) / p.nsplit + kDecodeTile - 1) / kDecodeTile * kDecodeTile);
  }
  const int t_begin = int(min(int64_t(split) * chunk, int64_t(len)));
  const int t_end = min(len, t_begin + chunk);
  const int ntiles = t_end > t_begin ? (t_end - t_begin + kTile - 1) / kTile : 0;

  // query heads as the B operand.  k-step m covers, for lane group g,
  //   int8: dims 16*(g + 4*(m/2)) + 8*(m%2) .. +7 in order
  //   int4: dims (d/4)*g + 8m + {0, 2, 4, 6, 1, 3, 5, 7}
  bf16x8 qf[KM];
  {
    const __bf16* qrow = p.q + (int64_t(b) * p.Hq + (head_ok ? hq : hk * p.G)) * D;
#pragma unroll
    for (int m = 0; m < KM; ++m) {
      const int d0 = BITS == 8 ? 16 * (g + 4 * (m >> 1)) + 8 * (m & 1) : (D / 4) * g + 8 * m;
      uint4 raw = *reinterpret_cast<const uint4*>(qrow + d0);
      if (!head_ok) raw = make_uint4(0u, 0u, 0u, 0u);
      const bf16x8 x = __builtin_bit_cast(bf16x8, raw);
      if constexpr (BITS == 8) {
        qf[m] = x;
      } else {
        qf[m] = __builtin_shufflevector(x, x, 0, 2, 4, 6, 1, 3, 5, 7);
      }
    }
  }

  // Tile loads (plain global loads into registers), issued three tiles ahead
  // of use.  Every load is unconditional: a token past the split end reads
  // the split's last token instead (its score is masked to -inf below, so its
  // probability is exactly 0 and its finite codes and scales add nothing).  A
  // load under a lane condition would become a branch, after which the
  // compiler can no longer count outstanding loads and waits for all of them
  // before every tile, which would empty the ring.
  const int v_row = lane / CPR, v_col = 16 * (lane % CPR);
  const float* sc_src = lane < kTile ? ksb : vsb;
  const int sc_tok = lane & (kTile - 1);
  auto load_tile = [&](int t, TileRegs<D, BITS>& r) __attribute__((always_inline)) {
    const int t0 = t_begin + t * kTile;
#pragma unroll
    for (int blk = 0; blk < 2; ++blk) {
      const int tok = min(t0 + 16 * blk + n, t_end - 1);
      const uint8_t* krow = kbase + int64_t(tok) * RB;
      if constexpr (BITS == 8) {
#pragma unroll
        for (int u = 0; u < KB / 16; ++u) load_k<16, NT>(krow + 16 * (g + 4 * u), &r.k[blk][4 * u]);
      } else {
        load_k<KB, NT>(krow + KB * g, r.k[blk]);
      }
    }
#pragma unroll
    for (int i = 0; i < VLOADS; ++i) {
      const int tok = min(t0 + i * RPL + v_row, t_end - 1);
      r.v[i] = load_stream16<NT>(vbase + int64_t(tok) * RB + v_col);
    }
    r.sc = load_stream4<NT>(sc_src + min(t0 + sc_tok, t_end - 1));
  };

  f32x4 acc[CB];
#pragma unroll
  for (int cb = 0; cb < CB; ++cb) acc[cb] = f32x4{};
  float m_run = kNegHuge, l_run = 0.f;

  // int4: the value operand carries +136 per element; pbias accumulates the
  // matching 136 * sum(p') and kbias is the score bias 136 * sum(q) of this
  // lane's head (every row of these products holds the same number).
  const bf16x8 c136 = __builtin_bit_cast(bf16x8, make_uint4(0x43084308u, 0x43084308u,
                                                            0x43084308u, 0x43084308u));
  f32x4 pbias = f32x4{};
  float kbias = 0.f;
  if constexpr (BITS == 4) {
    f32x4 kb = f32x4{};
#pragma unroll
    for (int m = 0; m < KM; ++m) kb = mfma16(c136, qf[m], kb);
    kbias = kb[0];
  }

  // P^T slot e of lane group g is token 4g + e (e < 4) or 16 + 4g + (e - 4);
  // source lane s of the group addresses that token's V row (tr8 read).
  const int s16 = lane & 15;
  const int e_src = s16 >> 1;
  const int vrow = e_src < 4 ? 4 * g + e_src : 16 + 4 * g + (e_src - 4);
  const char* vread = vlds + vrow * VSTRIDE + 8 * (s16 & 1);

  auto process = [&](int t, const TileRegs<D, BITS>& r) __attribute__((always_inline)) {
    const int t0 = t_begin + t * kTile;
    // stage V codes (row-major, padded rows) and the tile's scales
#pragma unroll
    for (int i = 0; i < VLOADS; ++i) {
      *reinterpret_cast<uint4*>(vlds + (i * RPL + v_row) * VSTRIDE + v_col) = r.v[i];
    }
    slds[lane] = r.sc;

    // S = K q^T: rows = tokens 16*blk + 4g + r, columns = head slot n
    f32x4 s[2];
#pragma unroll
    for (int blk = 0; blk < 2; ++blk) {
      s[blk] = f32x4{};
#pragma unroll
      for (int m = 0; m < KM; ++m) {
        bf16x8 a;
        if constexpr (BITS == 8) {
          a = i8x8_to_bf16x8(r.k[blk][2 * m], r.k[blk][2 * m + 1]);
        } else {  // 136 + code: even dims of the dword, then odd dims
          const uint32_t t4 = r.k[blk][m] ^ 0x88888888u;
          a = biased_bf16x8(t4 & 0x0f0f0f0fu, (t4 >> 4) & 0x0f0f0f0fu);
        }
        s[blk] = mfma16(a, qf[m], s[blk]);
      }
    }

    // scaled scores (base 2): the k scale of each token multiplies its score
    const f32x4 ks0 = *reinterpret_cast<const f32x4*>(slds + 4 * g);
    const f32x4 ks1 = *reinterpret_cast<const f32x4*>(slds + 16 + 4 * g);
    float tv[8];
#pragma unroll
    for (int rr = 0; rr < 4; ++rr) {
      tv[rr] = (s[0][rr] - kbias) * (ks0[rr] * p.c);
      tv[4 + rr] = (s[1][rr] - kbias) * (ks1[rr] * p.c);
    }
    if (t0 + kTile > t_end) {  // ragged last tile: tokens past the end are not keys
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        const int tok = t0 + (e < 4 ? 4 * g + e : 16 + 4 * g + (e - 4));
        if (tok >= t_end) tv[e] = -INFINITY;
      }
    }
    float mx = kNegHuge;
#pragma unroll
    for (int e = 0; e < 8; ++e) mx = fmaxf(mx, tv[e]);
    mx = wave_max_xor(mx, 16);
    mx = max_across_halves(mx);
    if (__builtin_expect(__any(mx > m_run + kLazy), 0)) {  // rare: raise the reference
      const float m_new = fmaxf(m_run, mx);
      const float alpha = __builtin_amdgcn_exp2f(m_run - m_new);
      m_run = m_new;
      l_run *= alpha;
#pragma unroll
      for (int cb = 0; cb < CB; ++cb) acc[cb] *= alpha;
      if constexpr (BITS == 4) pbias *= alpha;
    }
    const f32x4 vs0 = *reinterpret_cast<const f32x4*>(slds + kTile + 4 * g);
    const f32x4 vs1 = *reinterpret_cast<const f32x4*>(slds + kTile + 16 + 4 * g);
    float pv[8];
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      const float pe = __builtin_amdgcn_exp2f(tv[e] - m_run);
      l_run += pe;
      pv[e] = pe * (e < 4 ? vs0[e] : vs1[e - 4]);
    }
    const bf16x8 pf = to_bf16x8(pv[0], pv[1], pv[2], pv[3], pv[4], pv[5], pv[6], pv[7]);

    // O^T += V^T P^T with V^T read transposed from the staged tile
#pragma unroll
    for (int cb = 0; cb < GM::NREAD; ++cb) {
      const i32x2 raw = lds_read_tr8(vread + 16 * cb);
      const uint32_t r0w = uint32_t(raw[0]), r1w = uint32_t(raw[1]);
      if constexpr (BITS == 8) {
        acc[cb] = mfma16(i8x8_to_bf16x8(r0w, r1w), pf, acc[cb]);
      } else {  // byte column 16cb + t: even dim from the low nibbles, odd from the high
        const uint32_t t0 = r0w ^ 0x88888888u, t1 = r1w ^ 0x88888888u;
        acc[2 * cb] = mfma16(biased_bf16x8(t0 & 0x0f0f0f0fu, t1 & 0x0f0f0f0fu), pf, acc[2 * cb]);
        acc[2 * cb + 1] = mfma16(biased_bf16x8((t0 >> 4) & 0x0f0f0f0fu, (t1 >> 4) & 0x0f0f0f0fu),
                                 pf, acc[2 * cb + 1]);
      }
    }
    if constexpr (BITS == 4) pbias = mfma16(c136, pf, pbias);
  };

  // four-slot register ring: tiles t+1 .. t+3 are in flight while t is
  // processed.  Slots are refilled unconditionally (a tile past the end
  // rereads the split's last token, cached): with a fixed load sequence the
  // compiler waits only for the slot about to be used.
  // (An empty split, which the split plan never makes, skips the ring and
  // writes o = 0, lse = -inf below.)
  if (ntiles > 0) {
    constexpr int NS = kRingSlots;
    TileRegs<D, BITS> ring[NS];
#pragma unroll
    for (int j = 0; j < NS - 1; ++j) load_tile(j, ring[j]);
    for (int t = 0; t < ntiles; t += NS) {
#pragma unroll
      for (int j = 0; j < NS; ++j) {  // slot indices are compile-time after unrolling
        if (j > 0 && t + j >= ntiles) break;
        load_tile(t + j + NS - 1, ring[(j + NS - 1) % NS]);
        process(t + j, ring[j]);
      }
    }
  }

  // row sum over the four lane groups holding this head's tokens
  float l_tot = l_run + __shfl_xor(l_run, 16);
  l_tot += __shfl_xor(l_tot, 32);
  const float inv = l_tot > 0.f ? 1.f / l_tot : 0.f;
  const float lse_row = l_tot > 0.f ? m_run * kLn2 + logf(l_tot) : -INFINITY;
  if (p.nsplit == 1) {
    if (!head_ok) return;
    // a single split is the whole row: write the bf16 output and lse here
    // (what the merge would produce: weight exp(0) = 1, log 1 = 0)
    __bf16* orow = p.o + (int64_t(b) * p.Hq + hq) * D;
    if constexpr (BITS == 8) {
#pragma unroll
      for (int cb = 0; cb < CB; ++cb) {
        const f32x4 v = acc[cb] * inv;
        bf16x4 h;
        h[0] = (__bf16)v[0]; h[1] = (__bf16)v[1]; h[2] = (__bf16)v[2]; h[3] = (__bf16)v[3];
        *reinterpret_cast<bf16x4*>(orow + 16 * cb + 4 * g) = h;
      }
    } else {
#pragma unroll
      for (int cb = 0; cb < GM::NREAD; ++cb) {
        const f32x4 e = (acc[2 * cb] - pbias) * inv, o = (acc[2 * cb + 1] - pbias) * inv;
        *reinterpret_cast<bf16x8*>(orow + 32 * cb + 8 * g) =
            to_bf16x8(e[0], o[0], e[1], o[1], e[2], o[2], e[3], o[3]);
      }
    }
    if (g == 0 && p.lse) p.lse[int64_t(b) * p.Hq + hq] = lse_row;
    return;
  }

  // the normalised partial output of this split, written as 4-float pieces:
  // put(dim, f32x4) stores output dims dim .. dim+3 of head slot n
  auto write_partial = [&](auto put) __attribute__((always_inline)) {
    if constexpr (BITS == 8) {
#pragma unroll
      for (int cb = 0; cb < CB; ++cb) put(16 * cb + 4 * g, acc[cb] * inv);  // dims 16cb + 4g + r
    } else {
#pragma unroll
      for (int cb = 0; cb < GM::NREAD; ++cb) {
        // acc[2cb][r] / acc[2cb+1][r]: dims 32*cb + 8g + 2r and that + 1, each
        // carrying the bias 136 * sum(p') that pbias holds in every register
        const f32x4 e = (acc[2 * cb] - pbias) * inv, o = (acc[2 * cb + 1] - pbias) * inv;
        put(32 * cb + 8 * g, f32x4{e[0], o[0], e[1], o[1]});
        put(32 * cb + 8 * g + 4, f32x4{e[2], o[2], e[3], o[3]});
      }
    }
  };

  if constexpr (WG) {
    // Workgroup form: every wave (split) of the block leaves its partial in
    // LDS, over the staging areas (the barrier guarantees that no wave still
    // reads them), and the block merges in split order with the arithmetic
    // of decode_merge_kernel.
    const int hpw = min(kHeadsPerWave, p.G);  // head slots the merge area holds
    float* const mo = reinterpret_cast<float*>(dyn_lds);
    float* const ml = mo + p.nsplit * hpw * GM::MROW;
    __syncthreads();
    if (head_ok) {
      float* row = mo + (split * hpw + n) * GM::MROW;
      write_partial([&](int dim, const f32x4& v) __attribute__((always_inline)) {
        *reinterpret_cast<f32x4*>(row + dim) = v;
      });
      if (g == 0) ml[split * hpw + n] = lse_row;
    }
    __syncthreads();
    for (int idx = threadIdx.x; idx < nheads * D; idx += blockDim.x) {
      const int h = idx / D, c = idx % D;
      float mx = -INFINITY;
      for (int s2 = 0; s2 < p.nsplit; ++s2) mx = fmaxf(mx, ml[s2 * hpw + h]);
      float a = 0.f, wsum = 0.f;
      if (mx != -INFINITY) {
        for (int s2 = 0; s2 < p.nsplit; ++s2) {
          const float wgt = expf(ml[s2 * hpw + h] - mx);  // 0 for an empty split
          wsum += wgt;
          a = fmaf(wgt, mo[(s2 * hpw + h) * GM::MROW + c], a);
        }
      }
      const float winv = wsum > 0.f ? 1.f / wsum : 0.f;
      const int64_t orow = int64_t(b) * p.Hq + hk * p.G + head0 + h;
      p.o[orow * D + c] = (__bf16)(a * winv);
      if (c == 0 && p.lse) p.lse[orow] = wsum > 0.f ? mx + logf(wsum) : -INFINITY;
    }
    return;
  } else {
    if (!head_ok) return;
    const int64_t prow = (int64_t(b) * p.Hq + hq) * p.nsplit + split;
    float* po = p.part_o + prow * D;
    write_partial([&](int dim, const f32x4& v) __attribute__((always_inline)) {
      *reinterpret_cast<f32x4*>(po + dim) = v;
    });
    if (g == 0) p.part_lse[prow] = lse_row;
  }
}

// One wave per (batch, query head): merges nsplit partials by log-sum-exp.
template <int D>
__global__ __launch_bounds__(64) void decode_merge_kernel(const float* __restrict__ part_o,
                                                          const float* __restrict__ part_lse,
                                                          __bf16* __restrict__ o,
                                                          float* __restrict__ lse, int nsplit) {
  const int row = blockIdx.x;  // b * Hq + h
  const int lane = threadIdx.x;
  const float* pl = part_lse + int64_t(row) * nsplit;
  float mx = -INFINITY;
  for (int s = lane; s < nsplit; s += 64) mx = fmaxf(mx, pl[s]);
#pragma unroll
  for (int sh = 1; sh < 64; sh <<= 1) mx = fmaxf(mx, __shfl_xor(mx, sh));
  constexpr int PER = D / 64;
  float accv[PER];
#pragma unroll
  for (int i = 0; i < PER; ++i) accv[i] = 0.f;
  float wsum = 0.f;
  if (mx != -INFINITY) {
    const float* po = part_o + int64_t(row) * nsplit * D;
    for (int s = 0; s < nsplit; ++s) {
      const float w = expf(pl[s] - mx);  // 0 for an empty split
      wsum += w;
#pragma unroll
      for (int i = 0; i < PER; ++i) accv[i] = fmaf(w, po[int64_t(s) * D + lane + 64 * i], accv[i]);
    }
  }
  const float inv = wsum > 0.f ? 1.f / wsum : 0.f;
#pragma unroll
  for (int i = 0; i < PER; ++i) o[int64_t(row) * D + lane + 64 * i] = (__bf16)(accv[i] * inv);
  if (lse && lane == 0) lse[row] = wsum > 0.f ? mx + logf(wsum) : -INFINITY;
}

template <int D, int BITS, bool NT>
hipError_t launch_split_and_merge(const DecodeArgs& a, const SplitParams& p, hipStream_t stream) {
  const int64_t groups = int64_t(a.B) * a.Hkv * p.nhc;  // (b, kv head, head chunk)
  if (a.nsplit > 1 && a.nsplit <= kWgMaxSplits) {
    const int hpw = p.G < kHeadsPerWave ? p.G : kHeadsPerWave;
    return launch_kernel(decode_split_kernel<D, BITS, true, NT>, dim3(unsigned(groups)),
                         dim3(64 * a.nsplit), split_lds_bytes<D, BITS>(a.nsplit, hpw), stream, p);
  }
  hipError_t err = launch_kernel(decode_split_kernel<D, BITS, false, NT>,
                                 dim3(unsigned(groups * a.nsplit)), dim3(64),
                                 split_lds_bytes<D, BITS>(1, 0), stream, p);
  if (err != hipSuccess || a.nsplit == 1) return err;  // one split writes the output itself
  return launch_kernel(decode_merge_kernel<D>, dim3(unsigned(int64_t(a.B) * a.Hq)), dim3(64), 0,
                       stream, a.part_o, a.part_lse, static_cast<__bf16*>(a.o), a.lse, a.nsplit);
}

// the whole cache once: non-temporal loads; per-sequence lengths: plain loads
template <int D, int BITS>
hipError_t launch_split_and_merge(const DecodeArgs& a, const SplitParams& p, hipStream_t stream) {
  return a.seqlens ? launch_split_and_merge<D, BITS, false>(a, p, stream)
                   : launch_split_and_merge<D, BITS, true>(a, p, stream);
}

}  // namespace

// ---- built-in scratch for callers that cannot allocate.  The partial
// outputs and lse of plans that merge in a second kernel go here instead of
// a caller workspace (fattn_decode_int8_noalloc).  Nothing in it needs to
// start at zero: every partial is written before the merge reads it.  Every
// call on one GPU uses that GPU's copy, so calls that overlap on a GPU race.
static __device__ __align__(256) char scratch[kDecodeScratchBytes];

namespace {
constexpr int kMaxDevices = 256;
std::mutex g_scratch_mu;
void* g_scratch_ptr[kMaxDevices];  // device address of `scratch` per device, once taken
}  // namespace

hipError_t decode_scratch(hipStream_t stream, void** ptr) {
  // the GPU the kernels will run on: the stream's (the null stream is the
  // current device's)
  int dev = -1;
  hipError_t err = stream ? hipStreamGetDevice(stream, &dev) : hipGetDevice(&dev);
  if (err != hipSuccess) return err;
  if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (!g_scratch_ptr[dev]) {
    // the array's name is a host-side stand-in: only this address may be
    // handed to kernels (each device holds its own copy at its own address),
    // and it is taken with that device current
    int cur = -1;
    err = hipGetDevice(&cur);
    if (err != hipSuccess) return err;
    if (cur != dev && (err = hipSetDevice(dev)) != hipSuccess) return err;
    void* p = nullptr;
    err = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (cur != dev) {
      const hipError_t back = hipSetDevice(cur);
      if (err == hipSuccess) err = back;
    }
    if (err != hipSuccess) return err;
    if (!p) return hipErrorInvalidSymbol;
    g_scratch_ptr[dev] = p;
  }
  *ptr = g_scratch_ptr[dev];
  return hipSuccess;
}

hipError_t launch_decode(const DecodeArgs& a, hipStream_t stream) {
  SplitParams p;
  p.q = static_cast<const __bf16*>(a.q);
  p.kq = static_cast<const uint8_t*>(a.kq);
  p.ks = a.kscale;
  p.vq = static_cast<const uint8_t*>(a.vq);
  p.vs = a.vscale;
  p.part_o = a.part_o;
  p.part_lse = a.part_lse;
  p.o = static_cast<__bf16*>(a.o);
  p.lse = a.lse;
  p.seqlens = a.seqlens;
  p.Hq = a.Hq;
  p.Hkv = a.Hkv;
  p.Skv = a.Skv;
  p.G = a.Hq / a.Hkv;
  p.nhc = (p.G + kHeadsPerWave - 1) / kHeadsPerWave;
  p.nsplit = a.nsplit;
  p.chunk = a.chunk;
  p.c = a.scale * 1.4426950408889634f;
  const int64_t waves = int64_t(a.B) * a.Hkv * p.nhc * a.nsplit;
  const int64_t rows = int64_t(a.B) * a.Hq;
  if (waves > 0x7fffffff || rows > 0x7fffffff) return hipErrorInvalidConfiguration;
  if (a.bits != 8 && a.bits != 4) return hipErrorInvalidValue;
  if (a.d == 64) {
    return a.bits == 8 ? launch_split_and_merge<64, 8>(a, p, stream)
                       : launch_split_and_merge<64, 4>(a, p, stream);
  }
  return a.bits == 8 ? launch_split_and_merge<128, 8>(a, p, stream)
                     : launch_split_and_merge<128, 4>(a, p, stream);
}

}  // namespace fattn
