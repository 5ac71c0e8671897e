// Split-KV decode over an int8 KV cache, then a log-sum-exp merge.
//
// Method: one query token per sequence attends to all cached tokens.  The
// cache keeps int8 codes with an fp32 scale per (token, kv head) and is used
// without a decompressed copy ([FA-3MOVES] move 3): codes are converted to
// bf16 in registers (exact, |code| <= 127) and the scales are applied to the
// scores (k scale) and to the probabilities (v scale).  The keys of each
// (batch, kv head) stream are cut into splits; each split runs the online
// softmax of the [FA-NPU] tiling section over its tokens and writes a
// normalised partial output and its log-sum-exp; a second kernel merges the
// partials (global max of the partial lse, weights e^(lse_s - max)).
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
//    (about 25 KB in flight per wave), which is what keeps HBM busy: the
//    kernel is bound by bytes in flight, not by arithmetic.  Scales arrive as
//    one dword per lane per tile and are redistributed through LDS.
#include "device_util.h"
#include "launch.h"

#include <cmath>

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

struct SplitParams {
  const __bf16* q;
  const int8_t* kq;
  const float* ks;
  const int8_t* vq;
  const float* vs;
  float* part_o;
  float* part_lse;
  int Hq, Hkv, Skv;
  int G;        // query heads per kv head
  int nhc;      // head chunks per kv head: ceil(G / 16)
  int nsplit;
  int chunk;    // tokens per split
  float c;      // scale * log2(e)
};

// Loads of one 32-token tile held in registers between issue and use.
template <int D>
struct TileRegs {
  uint4 k[2][D / 64];   // K codes, MFMA A layout: token 16*blk + l%16, dims 16*(l/16 + 4u) ..
  uint4 v[D / 32];      // V codes, coalesced: 64 lanes x 16 bytes per load
  float sc;             // lane l < 32: k scale of token l; lane l >= 32: v scale of token l - 32
};

template <int D>
__global__ __launch_bounds__(64, 2) void decode_split_kernel(SplitParams p) {
  constexpr int KU = D / 64;              // 16-byte K pieces per token per lane group
  constexpr int KM = D / 32;              // k-steps of the QK product (32 dims each)
  constexpr int VLOADS = D / 32;          // 16-byte V loads per lane per tile
  constexpr int CPR = D / 16;             // 16-byte pieces per V row
  constexpr int RPL = 64 / CPR;           // V rows per load instruction
  constexpr int VSTRIDE = D + 16;         // padded LDS row (bytes)
  constexpr int CB = D / 16;              // 16-dim blocks of the output
  __shared__ __attribute__((aligned(16))) char vlds[kTile * VSTRIDE];
  __shared__ __attribute__((aligned(16))) float slds[2 * kTile];   // k scales, then v scales

  const int lane = threadIdx.x;
  const int n = lane & 15;   // head slot (B/C column), also token row of A
  const int g = lane >> 4;   // lane group

  int id = blockIdx.x;
  const int split = id % p.nsplit; id /= p.nsplit;
  const int hc = id % p.nhc; id /= p.nhc;
  const int hk = id % p.Hkv;
  const int b = id / p.Hkv;
  const int head0 = hc * kHeadsPerWave;
  const int nheads = min(kHeadsPerWave, p.G - head0);
  const int hq = hk * p.G + head0 + n;      // this lane's query head (if n < nheads)
  const bool head_ok = n < nheads;

  const int64_t stream = int64_t(b) * p.Hkv + hk;
  const int8_t* kbase = p.kq + stream * p.Skv * D;
  const int8_t* vbase = p.vq + stream * p.Skv * D;
  const float* ksb = p.ks + stream * p.Skv;
  const float* vsb = p.vs + stream * p.Skv;

  const int t_begin = split * p.chunk;
  const int t_end = min(p.Skv, t_begin + p.chunk);
  const int ntiles = t_end > t_begin ? (t_end - t_begin + kTile - 1) / kTile : 0;

  // query heads as the B operand: k-step m covers dims 16*(g + 4*(m/2)) + 8*(m%2) .. +7
  bf16x8 qf[KM];
  {
    const __bf16* qrow = p.q + (int64_t(b) * p.Hq + (head_ok ? hq : hk * p.G)) * D;
#pragma unroll
    for (int m = 0; m < KM; ++m) {
      const int d0 = 16 * (g + 4 * (m >> 1)) + 8 * (m & 1);
      uint4 raw = *reinterpret_cast<const uint4*>(qrow + d0);
      if (!head_ok) raw = make_uint4(0u, 0u, 0u, 0u);
      qf[m] = __builtin_bit_cast(bf16x8, raw);
    }
  }

  // Tile loads (plain global loads into registers; tokens past the split end
  // read as zero).  Issued three tiles ahead of use.
  const int v_row = lane / CPR, v_col = 16 * (lane % CPR);
  const float* sc_src = lane < kTile ? ksb : vsb;
  const int sc_tok = lane & (kTile - 1);
  auto load_tile = [&](int t, TileRegs<D>& r) __attribute__((always_inline)) {
    const int t0 = t_begin + t * kTile;
#pragma unroll
    for (int blk = 0; blk < 2; ++blk) {
      const int tok = t0 + 16 * blk + n;
#pragma unroll
      for (int u = 0; u < KU; ++u) {
        r.k[blk][u] = tok < t_end
            ? *reinterpret_cast<const uint4*>(kbase + int64_t(tok) * D + 16 * (g + 4 * u))
            : make_uint4(0u, 0u, 0u, 0u);
      }
    }
#pragma unroll
    for (int i = 0; i < VLOADS; ++i) {
      const int tok = t0 + i * RPL + v_row;
      r.v[i] = tok < t_end ? *reinterpret_cast<const uint4*>(vbase + int64_t(tok) * D + v_col)
                           : make_uint4(0u, 0u, 0u, 0u);
    }
    const int stok = t0 + sc_tok;
    r.sc = stok < t_end ? sc_src[stok] : 0.f;
  };

  f32x4 acc[CB];
#pragma unroll
  for (int cb = 0; cb < CB; ++cb) acc[cb] = f32x4{};
  float m_run = kNegHuge, l_run = 0.f;

  // P^T slot e of lane group g is token 4g + e (e < 4) or 16 + 4g + (e - 4);
  // source lane s of the group addresses that token's V row (tr8 read).
  const int s16 = lane & 15;
  const int e_src = s16 >> 1;
  const int vrow = e_src < 4 ? 4 * g + e_src : 16 + 4 * g + (e_src - 4);
  const char* vread = vlds + vrow * VSTRIDE + 8 * (s16 & 1);

  auto process = [&](int t, const TileRegs<D>& r) __attribute__((always_inline)) {
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
        const uint4 w = r.k[blk][m >> 1];
        const bf16x8 a = (m & 1) ? i8x8_to_bf16x8(w.z, w.w) : i8x8_to_bf16x8(w.x, w.y);
        s[blk] = mfma16(a, qf[m], s[blk]);
      }
    }

    // scaled scores (base 2): the k scale of each token multiplies its score
    const f32x4 ks0 = *reinterpret_cast<const f32x4*>(slds + 4 * g);
    const f32x4 ks1 = *reinterpret_cast<const f32x4*>(slds + 16 + 4 * g);
    float tv[8];
#pragma unroll
    for (int rr = 0; rr < 4; ++rr) {
      tv[rr] = s[0][rr] * (ks0[rr] * p.c);
      tv[4 + rr] = s[1][rr] * (ks1[rr] * p.c);
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
    for (int cb = 0; cb < CB; ++cb) {
      const i32x2 raw = lds_read_tr8(vread + 16 * cb);
      const bf16x8 a = i8x8_to_bf16x8(uint32_t(raw[0]), uint32_t(raw[1]));
      acc[cb] = mfma16(a, pf, acc[cb]);
    }
  };

  // four-slot register ring: tiles t+1 .. t+3 are in flight while t is processed
  TileRegs<D> r0, r1, r2, r3;
  if (0 < ntiles) load_tile(0, r0);
  if (1 < ntiles) load_tile(1, r1);
  if (2 < ntiles) load_tile(2, r2);
  for (int t = 0; t < ntiles; t += 4) {
    if (t + 3 < ntiles) load_tile(t + 3, r3);
    process(t, r0);
    if (t + 1 >= ntiles) break;
    if (t + 4 < ntiles) load_tile(t + 4, r0);
    process(t + 1, r1);
    if (t + 2 >= ntiles) break;
    if (t + 5 < ntiles) load_tile(t + 5, r1);
    process(t + 2, r2);
    if (t + 3 >= ntiles) break;
    if (t + 6 < ntiles) load_tile(t + 6, r2);
    process(t + 3, r3);
  }

  // row sum over the four lane groups holding this head's tokens
  float l_tot = l_run + __shfl_xor(l_run, 16);
  l_tot += __shfl_xor(l_tot, 32);
  if (!head_ok) return;
  const float inv = l_tot > 0.f ? 1.f / l_tot : 0.f;
  const int64_t prow = (int64_t(b) * p.Hq + hq) * p.nsplit + split;
  float* po = p.part_o + prow * D;
#pragma unroll
  for (int cb = 0; cb < CB; ++cb) {
    // acc[cb][r] holds output dim 16*cb + 4g + r of head slot n
    *reinterpret_cast<f32x4*>(po + 16 * cb + 4 * g) = acc[cb] * inv;
  }
  if (g == 0) p.part_lse[prow] = l_tot > 0.f ? m_run * kLn2 + logf(l_tot) : -INFINITY;
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

}  // namespace

hipError_t launch_decode_int8(const DecodeArgs& a, hipStream_t stream) {
  SplitParams p;
  p.q = static_cast<const __bf16*>(a.q);
  p.kq = a.kq;
  p.ks = a.kscale;
  p.vq = a.vq;
  p.vs = a.vscale;
  p.part_o = a.part_o;
  p.part_lse = a.part_lse;
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
  if (a.d == 64) {
    hipLaunchKernelGGL(decode_split_kernel<64>, dim3(unsigned(waves)), dim3(64), 0, stream, p);
    hipLaunchKernelGGL(decode_merge_kernel<64>, dim3(unsigned(rows)), dim3(64), 0, stream,
                       a.part_o, a.part_lse, static_cast<__bf16*>(a.o), a.lse, a.nsplit);
  } else {
    hipLaunchKernelGGL(decode_split_kernel<128>, dim3(unsigned(waves)), dim3(64), 0, stream, p);
    hipLaunchKernelGGL(decode_merge_kernel<128>, dim3(unsigned(rows)), dim3(64), 0, stream,
                       a.part_o, a.part_lse, static_cast<__bf16*>(a.o), a.lse, a.nsplit);
  }
  return hipGetLastError();
}

}  // namespace fattn
