// fp32 tiled exact attention (vector ALU), for float32 inputs.
//
// One wave (64 lanes) per block of 64 query positions of one query head; each
// lane owns one query row.  Key/value tiles of 32 rows are staged through LDS
// and read by all lanes as broadcasts.  Per tile every lane computes its 32
// scores, then applies the online softmax of the [FA-NPU] tiling section and
// [FA-3MOVES] move 2: running max m and running sum l per row, the
// accumulator rescaled by exp(m_old - m_new) when the max grows.  The score
// matrix lives only in registers.
//
// Arithmetic: fp32 dot products (fma chains in index order), exp via expf on
// scale * s - m, fp32 accumulation; lse = m + log(l).
#include "device_util.h"
#include "launch.h"

#include <cmath>

namespace fattn {
namespace {

constexpr int kRows = 64;      // query positions per block (one per lane)
constexpr int kTile = 32;      // keys per LDS tile
constexpr float kNegHuge = -1e30f;  // finite start value of the running max

template <int D>
__global__ __launch_bounds__(64) void fwd_f32_kernel(const float* __restrict__ q,
                                                     const float* __restrict__ k,
                                                     const float* __restrict__ v,
                                                     float* __restrict__ o,
                                                     float* __restrict__ lse,
                                                     int Hq, int Hkv, int Sq, int Skv,
                                                     float scale, int causal, int window,
                                                     const int* __restrict__ cu_q,
                                                     const int* __restrict__ cu_k,
                                                     int total_q, int total_k) {
  __shared__ float4 ks[kTile * D / 4];
  __shared__ float4 vs[kTile * D / 4];

  const int lane = threadIdx.x;
  // blockIdx.x enumerates (query block, head, batch), query block fastest;
  // Sq / Skv are the (longest) sequence lengths the grid was sized for
  const int nqb = (Sq + kRows - 1) / kRows;
  const int qblk = int(blockIdx.x % unsigned(nqb));
  const int bh = int(blockIdx.x / unsigned(nqb));
  const int h = bh % Hq;
  const int b = bh / Hq;
  const int hk = h / (Hq / Hkv);
  const int p0 = qblk * kRows;
  const SeqView sv = seq_view(cu_q, cu_k, total_q, total_k, b, Hq, Sq, Skv);
  Sq = sv.Sq;
  Skv = sv.Skv;
  if (p0 >= Sq) return;  // a row block past this sequence's end (block-uniform)
  const int i = p0 + lane;
  const bool active = i < Sq;
  const int64_t off = int64_t(Skv) - Sq;

  // visible key range of this lane's row, and of the whole block
  int64_t row_hi = Skv, row_lo = 0;
  int64_t blk_hi = Skv, blk_lo = 0;
  if (causal) {
    const int64_t p_last = (p0 + kRows - 1 < Sq ? p0 + kRows - 1 : Sq - 1);
    row_hi = i + off + 1;
    blk_hi = p_last + off + 1;
    if (window > 0) {
      row_lo = i + off - window + 1;
      blk_lo = p0 + off - window + 1;
    }
  }
  if (row_hi > Skv) row_hi = Skv;
  if (blk_hi > Skv) blk_hi = Skv;
  if (row_lo < 0) row_lo = 0;
  if (blk_lo < 0) blk_lo = 0;

  float qr[D];
  float acc[D];
  const float* qp = q + ((sv.q_row0 + (active ? i : 0)) * Hq + h) * D;
#pragma unroll
  for (int c = 0; c < D; c += 4) {
    float4 t = *reinterpret_cast<const float4*>(qp + c);
    qr[c] = t.x; qr[c + 1] = t.y; qr[c + 2] = t.z; qr[c + 3] = t.w;
  }
#pragma unroll
  for (int c = 0; c < D; ++c) acc[c] = 0.f;
  float m = kNegHuge, l = 0.f;

  const int64_t kv_row = int64_t(Hkv) * D;  // elements between consecutive keys
  const float* kb = k + (sv.k_row0 * Hkv + hk) * D;
  const float* vb = v + (sv.k_row0 * Hkv + hk) * D;

  for (int64_t j0 = blk_lo; j0 < blk_hi; j0 += kTile) {
    __syncthreads();
    // stage K/V rows j0 .. j0+kTile-1 (zero rows past the end)
    for (int e = lane; e < kTile * D / 4; e += 64) {
      const int r = e / (D / 4), c4 = e % (D / 4);
      const int64_t j = j0 + r;
      float4 kk = make_float4(0.f, 0.f, 0.f, 0.f), vv = kk;
      if (j < blk_hi) {
        kk = *reinterpret_cast<const float4*>(kb + j * kv_row + 4 * c4);
        vv = *reinterpret_cast<const float4*>(vb + j * kv_row + 4 * c4);
      }
      ks[e] = kk;
      vs[e] = vv;
    }
    __syncthreads();

    float s[kTile];
    float tmax = kNegHuge;
#pragma unroll
    for (int jj = 0; jj < kTile; ++jj) {
      const float4* kr = ks + jj * (D / 4);
      float dot = 0.f;
#pragma unroll
      for (int c4 = 0; c4 < D / 4; ++c4) {
        float4 t = kr[c4];
        dot = fmaf(qr[4 * c4], t.x, dot);
        dot = fmaf(qr[4 * c4 + 1], t.y, dot);
        dot = fmaf(qr[4 * c4 + 2], t.z, dot);
        dot = fmaf(qr[4 * c4 + 3], t.w, dot);
      }
      const int64_t j = j0 + jj;
      const bool vis = j >= row_lo && j < row_hi;
      s[jj] = vis ? dot * scale : -INFINITY;
      tmax = fmaxf(tmax, s[jj]);
    }
    const float m_new = fmaxf(m, tmax);
    const float alpha = expf(m - m_new);
    l *= alpha;
#pragma unroll
    for (int c = 0; c < D; ++c) acc[c] *= alpha;
    m = m_new;
#pragma unroll
    for (int jj = 0; jj < kTile; ++jj) {
      const float p = expf(s[jj] - m);  // exp(-inf) = 0 for masked keys
      l += p;
      const float4* vr = vs + jj * (D / 4);
#pragma unroll
      for (int c4 = 0; c4 < D / 4; ++c4) {
        float4 t = vr[c4];
        acc[4 * c4] = fmaf(p, t.x, acc[4 * c4]);
        acc[4 * c4 + 1] = fmaf(p, t.y, acc[4 * c4 + 1]);
        acc[4 * c4 + 2] = fmaf(p, t.z, acc[4 * c4 + 2]);
        acc[4 * c4 + 3] = fmaf(p, t.w, acc[4 * c4 + 3]);
      }
    }
  }

  if (!active) return;
  float* op = o + ((sv.q_row0 + i) * Hq + h) * D;
  const float inv = l > 0.f ? 1.f / l : 0.f;
#pragma unroll
  for (int c = 0; c < D; c += 4) {
    *reinterpret_cast<float4*>(op + c) =
        make_float4(acc[c] * inv, acc[c + 1] * inv, acc[c + 2] * inv, acc[c + 3] * inv);
  }
  if (lse) lse[sv.lse0 + int64_t(h) * sv.lse_hs + i] = l > 0.f ? m + logf(l) : -INFINITY;
}

}  // namespace

hipError_t launch_fwd_f32(const FwdArgs& a, hipStream_t stream) {
  const int64_t blocks = int64_t((a.Sq + kRows - 1) / kRows) * a.Hq * a.B;
  if (blocks > 0x7fffffff) return hipErrorInvalidConfiguration;
  const dim3 grid{unsigned(blocks), 1u, 1u};
  const float* q = static_cast<const float*>(a.q);
  const float* k = static_cast<const float*>(a.k);
  const float* v = static_cast<const float*>(a.v);
  float* o = static_cast<float*>(a.o);
  return launch_kernel(a.d == 64 ? fwd_f32_kernel<64> : fwd_f32_kernel<128>, grid, dim3(64), 0,
                       stream, q, k, v, o, a.lse, a.Hq, a.Hkv, a.Sq, a.Skv, a.scale, a.causal,
                       a.window, a.cu_q, a.cu_k, a.total_q, a.total_k);
}

}  // namespace fattn
