// C-ABI layer of libfattn: argument validation, split planning, dispatch.
//
// Validation runs before any HIP call, so an invalid call enqueues nothing and
// writes nothing, and this part is testable on a machine without a GPU.
#include "fattn.h"
#include "launch.h"

#include <cmath>
#include <cstddef>
#include <cstdint>

namespace {

constexpr int kVersion = 10000;  // 1.0.0

// Largest element count a tensor may have: offsets are computed in 64-bit
// arithmetic and must not overflow when multiplied by the element size.
constexpr int64_t kMaxElements = int64_t(1) << 56;

bool fits(int64_t a, int64_t b, int64_t c, int64_t d) {
  // a*b*c*d <= kMaxElements, with every factor >= 1
  int64_t p = a;
  for (int64_t f : {b, c, d}) {
    if (p > kMaxElements / f) return false;
    p *= f;
  }
  return true;
}

bool supported_head_dim(int d) { return d == 64 || d == 128; }

// Kernels use 16-byte vector loads/stores on every tensor.
bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }
bool aligned4(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 3u) == 0; }

// Automatic split count.  The split kernel runs one wave per (b, kv head,
// chunk of <= 16 query heads, split) at up to two waves per SIMD, so MI355X
// holds 256 CUs x 4 SIMDs x 2 = 2048 of them at once.  Measured on MI355X with
// the B=32, Hkv=8, 32K-token cache: a partial second round of waves leaves
// most of the chip idle while it drains (9 or 10 splits run 25-30% slower
// than 8); one wave per SIMD (4 splits) is 2-5% faster on an idle chip but
// 12% slower right after a prefill kernel, where two waves per SIMD hide the
// slower start.  So the count is the largest that keeps all waves in one
// round of 2048, with each split >= 256 tokens.  A pure function of the
// arguments (no device query), so the workspace size is known on the host
// before any device work.
int auto_splits(int B, int Hq, int Hkv, int Skv) {
  const int64_t resident_waves = 2048;
  const int64_t head_chunks = (int64_t(Hq / Hkv) + 15) / 16;
  const int64_t per_split = int64_t(B) * Hkv * head_chunks;
  int64_t want = resident_waves / per_split;
  const int64_t max_by_len = (int64_t(Skv) + 255) / 256;
  if (want > max_by_len) want = max_by_len;
  if (want < 1) want = 1;
  if (want > 1024) want = 1024;
  return int(want);
}

// Resolves the split plan: chunk = tokens per split (a multiple of the kernel
// tile), nsplit = number of non-empty splits.
void plan_splits(int B, int Hq, int Hkv, int Skv, int requested, int* nsplit, int* chunk) {
  int want = requested > 0 ? requested : auto_splits(B, Hq, Hkv, Skv);
  if (want > Skv) want = Skv;
  int64_t c = (int64_t(Skv) + want - 1) / want;
  c = (c + fattn::kDecodeTile - 1) / fattn::kDecodeTile * fattn::kDecodeTile;
  *chunk = int(c);
  *nsplit = int((int64_t(Skv) + c - 1) / c);
}

int validate_decode(const void* q, const void* kq, const void* ks, const void* vq, const void* vs,
                    const void* o, int B, int Hq, int Hkv, int Skv, int d, float scale,
                    int num_splits, bool check_pointers) {
  if (check_pointers && (!q || !kq || !ks || !vq || !vs || !o)) return FATTN_EINVAL;
  if (check_pointers && !(aligned16(q) && aligned16(kq) && aligned16(ks) && aligned16(vq) &&
                          aligned16(vs) && aligned16(o)))
    return FATTN_EINVAL;
  if (B < 1 || Hq < 1 || Hkv < 1 || Skv < 1 || d < 1) return FATTN_EINVAL;
  if (Hq % Hkv != 0) return FATTN_EINVAL;
  if (!std::isfinite(scale)) return FATTN_EINVAL;
  if (num_splits < 0) return FATTN_EINVAL;
  if (!fits(B, Hkv, Skv, d) || !fits(B, Hq, d, 1)) return FATTN_EINVAL;
  if (!supported_head_dim(d)) return FATTN_EUNSUPPORTED;
  return FATTN_OK;
}

// Backward workspace: lse * log2(e) then D, each [B, Hq, Sq] fp32; then, if
// the dK/dV kernel splits the query heads of a group, fp32 partial dK and dV
// [nsplit, B, Skv, Hkv, d]; every part rounded up to 256 bytes.
size_t round256(size_t n) { return (n + 255) / 256 * 256; }
size_t bwd_stat_bytes(int B, int Hq, int Sq) {
  return round256(size_t(B) * size_t(Hq) * size_t(Sq) * sizeof(float));
}
size_t bwd_part_bytes(int B, int Hq, int Hkv, int Skv, int d) {
  const int ns = fattn::bwd_head_splits(B, Hq, Hkv, Skv);
  if (ns <= 1) return 0;
  return round256(size_t(ns) * size_t(B) * size_t(Skv) * size_t(Hkv) * size_t(d) * sizeof(float));
}
size_t bwd_workspace_bytes(int B, int Hq, int Hkv, int Sq, int Skv, int d) {
  return 2 * bwd_stat_bytes(B, Hq, Sq) + 2 * bwd_part_bytes(B, Hq, Hkv, Skv, d);
}

size_t workspace_bytes_for(int B, int Hq, int nsplit, int d) {
  // partial outputs [B, Hq, nsplit, d] fp32, then partial lse [B, Hq, nsplit]
  // fp32, the second array starting on a 256-byte boundary.
  size_t rows = size_t(B) * size_t(Hq) * size_t(nsplit);
  size_t o_bytes = (rows * size_t(d) * sizeof(float) + 255) / 256 * 256;
  return o_bytes + rows * sizeof(float);
}

// workspace == kBuiltinScratch: the library's own scratch array instead of a
// caller workspace (fattn_decode_int8_noalloc).
void* const kBuiltinScratch = reinterpret_cast<void*>(uintptr_t(1));

int decode(const void* q, const void* kq, const float* k_scale, const void* vq,
           const float* v_scale, void* o, float* lse, int B, int Hq, int Hkv, int Skv, int d,
           float scale, int num_splits, void* workspace, size_t workspace_bytes, void* stream,
           int bits, const int* seqlens = nullptr, bool varlen = false) {
  int st = validate_decode(q, kq, k_scale, vq, v_scale, o, B, Hq, Hkv, Skv, d, scale,
                           num_splits, true);
  if (st != FATTN_OK) return st;
  if (varlen && (!seqlens || !aligned4(seqlens))) return FATTN_EINVAL;
  if (lse && !aligned16(lse)) return FATTN_EINVAL;
  int nsplit, chunk;
  plan_splits(B, Hq, Hkv, Skv, num_splits, &nsplit, &chunk);
  size_t need = workspace_bytes_for(B, Hq, nsplit, d);
  if (workspace == kBuiltinScratch) {
    if (need > fattn::kDecodeScratchBytes) return FATTN_EWORKSPACE;
    // only plans that merge through partials touch memory beyond o and lse
    workspace = nullptr;
    if (nsplit > fattn::kDecodeWgMaxSplits) {
      if (fattn::decode_scratch(static_cast<hipStream_t>(stream), &workspace) != hipSuccess) return FATTN_EHIP;
    }
  } else if (!workspace || workspace_bytes < need || !aligned16(workspace)) {
    return FATTN_EWORKSPACE;
  }

  size_t rows = size_t(B) * size_t(Hq) * size_t(nsplit);
  size_t o_bytes = (rows * size_t(d) * sizeof(float) + 255) / 256 * 256;
  float* part_o = static_cast<float*>(workspace);
  float* part_lse = workspace ? reinterpret_cast<float*>(static_cast<char*>(workspace) + o_bytes)
                              : nullptr;
  fattn::DecodeArgs a{q, kq, k_scale, vq, v_scale, o, lse, B, Hq, Hkv, Skv, d, scale,
                      nsplit, chunk, part_o, part_lse, bits, seqlens};
  hipError_t err = fattn::launch_decode(a, static_cast<hipStream_t>(stream));
  return err == hipSuccess ? FATTN_OK : FATTN_EHIP;
}

int kv_append(const void* x, void* codes, float* scales, int B, int T, int Hkv, int d, int pos,
              int cap, int dtype, void* stream, int bits) {
  if (!x || !codes || !scales) return FATTN_EINVAL;
  if (!aligned16(x) || !aligned16(codes) || !aligned16(scales)) return FATTN_EINVAL;
  if (B < 1 || T < 1 || Hkv < 1 || d < 1 || pos < 0 || cap < 1) return FATTN_EINVAL;
  if (int64_t(pos) + T > cap) return FATTN_EINVAL;
  if (!fits(B, T, Hkv, d) || !fits(B, Hkv, cap, d)) return FATTN_EINVAL;
  if (int64_t(B) * T * Hkv > int64_t(0x7fffffff) * 16) return FATTN_EINVAL;
  if (dtype != FATTN_F32 && dtype != FATTN_BF16) return FATTN_EUNSUPPORTED;
  if (!supported_head_dim(d)) return FATTN_EUNSUPPORTED;
  fattn::KvQuantArgs a{x, codes, scales, B, T, Hkv, d, pos, cap, dtype == FATTN_BF16, bits};
  hipError_t err = fattn::launch_kv_quant(a, static_cast<hipStream_t>(stream));
  return err == hipSuccess ? FATTN_OK : FATTN_EHIP;
}

}  // namespace

extern "C" {

int fattn_fwd(const void* q, const void* k, const void* v, void* o, float* lse,
              int B, int Hq, int Hkv, int Sq, int Skv, int d,
              float scale, int causal, int window, int dtype, void* stream) {
  if (!q || !k || !v || !o) return FATTN_EINVAL;
  if (!aligned16(q) || !aligned16(k) || !aligned16(v) || !aligned16(o)) return FATTN_EINVAL;
  if (lse && !aligned16(lse)) return FATTN_EINVAL;
  if (B < 1 || Hq < 1 || Hkv < 1 || Sq < 1 || Skv < 1 || d < 1) return FATTN_EINVAL;
  if (Hq % Hkv != 0) return FATTN_EINVAL;
  if (!std::isfinite(scale)) return FATTN_EINVAL;
  if (causal != 0 && causal != 1) return FATTN_EINVAL;
  if (window < 0 || (window > 0 && !causal)) return FATTN_EINVAL;
  if (!fits(B, Sq, Hq, d) || !fits(B, Skv, Hkv, d)) return FATTN_EINVAL;
  // the kernels use one-dimensional grids of at most B*Hq*ceil(Sq/4) blocks
  if (int64_t(B) * Hq * ((int64_t(Sq) + 3) / 4) > 0x7fffffff) return FATTN_EINVAL;
  // offsets inside a 64-key tile (64 rows of Hkv*d elements) are 32-bit, and
  // so are the byte offsets of a block's output rows (128 rows of Hq*d)
  if (int64_t(Hkv) * d * 64 > 0x7fffffff) return FATTN_EINVAL;
  if (int64_t(Hq) * d * 256 > 0xffffffffll) return FATTN_EINVAL;
  if (dtype != FATTN_F32 && dtype != FATTN_BF16) return FATTN_EUNSUPPORTED;
  if (!supported_head_dim(d)) return FATTN_EUNSUPPORTED;

  fattn::FwdArgs a{q, k, v, o, lse, B, Hq, Hkv, Sq, Skv, d, scale, causal, window};
  hipStream_t s = static_cast<hipStream_t>(stream);
  hipError_t err = dtype == FATTN_F32 ? fattn::launch_fwd_f32(a, s) : fattn::launch_fwd_bf16(a, s);
  return err == hipSuccess ? FATTN_OK : FATTN_EHIP;
}

int fattn_fwd_varlen(const void* q, const void* k, const void* v, void* o, float* lse,
                     const int* cu_seqlens_q, const int* cu_seqlens_k, int B, int Hq, int Hkv,
                     int total_q, int total_k, int max_seqlen_q, int d, float scale, int causal,
                     int window, int dtype, void* stream) {
  // empty tensors may come with null pointers: q/o are only needed when there
  // are query rows, k/v only when there are keys
  if (B < 1 || Hq < 1 || Hkv < 1 || total_q < 0 || total_k < 0 || d < 1) return FATTN_EINVAL;
  if (!cu_seqlens_q || !cu_seqlens_k) return FATTN_EINVAL;
  if ((total_q > 0 && (!q || !o)) || (total_k > 0 && (!k || !v))) return FATTN_EINVAL;
  if (!aligned16(q) || !aligned16(k) || !aligned16(v) || !aligned16(o)) return FATTN_EINVAL;
  if (!aligned4(cu_seqlens_q) || !aligned4(cu_seqlens_k) || (lse && !aligned4(lse))) return FATTN_EINVAL;
  if (Hq % Hkv != 0) return FATTN_EINVAL;
  if (max_seqlen_q < 0 || max_seqlen_q > total_q || (total_q > 0 && max_seqlen_q < 1)) return FATTN_EINVAL;
  if (!std::isfinite(scale)) return FATTN_EINVAL;
  if (causal != 0 && causal != 1) return FATTN_EINVAL;
  if (window < 0 || (window > 0 && !causal)) return FATTN_EINVAL;
  if (!fits(total_q, Hq, d, 1) || !fits(total_k, Hkv, d, 1)) return FATTN_EINVAL;
  if (int64_t(B) * Hq * ((int64_t(max_seqlen_q) + 3) / 4) > 0x7fffffff) return FATTN_EINVAL;
  if (int64_t(Hkv) * d * 64 > 0x7fffffff) return FATTN_EINVAL;  // 32-bit offsets in a key tile
  if (int64_t(Hq) * d * 256 > 0xffffffffll) return FATTN_EINVAL;  // ... and in a block's output rows
  if (dtype != FATTN_F32 && dtype != FATTN_BF16) return FATTN_EUNSUPPORTED;
  if (!supported_head_dim(d)) return FATTN_EUNSUPPORTED;
  if (total_q == 0) return FATTN_OK;  // no query rows: nothing to compute

  fattn::FwdArgs a{q, k, v, o, lse, B, Hq, Hkv, max_seqlen_q, total_k, d, scale, causal, window,
                   cu_seqlens_q, cu_seqlens_k, total_q, total_k};
  hipStream_t s = static_cast<hipStream_t>(stream);
  hipError_t err = dtype == FATTN_F32 ? fattn::launch_fwd_f32(a, s) : fattn::launch_fwd_bf16(a, s);
  return err == hipSuccess ? FATTN_OK : FATTN_EHIP;
}

size_t fattn_bwd_workspace_size(int B, int Hq, int Hkv, int Sq, int Skv, int d) {
  if (B < 1 || Hq < 1 || Hkv < 1 || Sq < 1 || Skv < 1 || Hq % Hkv != 0) return 0;
  if (!fits(B, Hq, Sq, 1) || !fits(B, Skv, Hkv, d) || !supported_head_dim(d)) return 0;
  return bwd_workspace_bytes(B, Hq, Hkv, Sq, Skv, d);
}

int fattn_bwd(const void* q, const void* k, const void* v, const void* o, const float* lse,
              const void* dout, void* dq, void* dk, void* dv, int B, int Hq, int Hkv, int Sq,
              int Skv, int d, float scale, int causal, int window, int dtype, void* workspace,
              size_t workspace_bytes, void* stream) {
  if (!q || !k || !v || !o || !lse || !dout || !dq || !dk || !dv) return FATTN_EINVAL;
  if (!aligned16(q) || !aligned16(k) || !aligned16(v) || !aligned16(o) || !aligned16(lse) ||
      !aligned16(dout) || !aligned16(dq) || !aligned16(dk) || !aligned16(dv))
    return FATTN_EINVAL;
  if (B < 1 || Hq < 1 || Hkv < 1 || Sq < 1 || Skv < 1 || d < 1) return FATTN_EINVAL;
  if (Hq % Hkv != 0) return FATTN_EINVAL;
  if (!std::isfinite(scale)) return FATTN_EINVAL;
  if (causal != 0 && causal != 1) return FATTN_EINVAL;
  if (window < 0 || (window > 0 && !causal)) return FATTN_EINVAL;
  if (!fits(B, Sq, Hq, d) || !fits(B, Skv, Hkv, d)) return FATTN_EINVAL;
  if (int64_t(B) * Hq * ((int64_t(Sq) + 3) / 4) > 0x7fffffff) return FATTN_EINVAL;
  if (int64_t(B) * Hkv * ((int64_t(Skv) + 127) / 128) > 0x7fffffff) return FATTN_EINVAL;
  if (int64_t(Hq) * d * 256 > 0xffffffffll) return FATTN_EINVAL;  // 32-bit offsets of a block's rows
  if (dtype != FATTN_BF16) return FATTN_EUNSUPPORTED;
  if (!supported_head_dim(d)) return FATTN_EUNSUPPORTED;
  if (!workspace || !aligned16(workspace) ||
      workspace_bytes < bwd_workspace_bytes(B, Hq, Hkv, Sq, Skv, d))
    return FATTN_EWORKSPACE;
  char* ws = static_cast<char*>(workspace);
  const size_t st = bwd_stat_bytes(B, Hq, Sq), pt = bwd_part_bytes(B, Hq, Hkv, Skv, d);
  fattn::BwdArgs a{q, k, v, o, lse, dout, dq, dk, dv, B, Hq, Hkv, Sq, Skv, d, scale, causal, window,
                   reinterpret_cast<float*>(ws), reinterpret_cast<float*>(ws + st),
                   pt ? reinterpret_cast<float*>(ws + 2 * st) : nullptr,
                   pt ? reinterpret_cast<float*>(ws + 2 * st + pt) : nullptr};
  hipError_t err = fattn::launch_bwd_bf16(a, static_cast<hipStream_t>(stream));
  return err == hipSuccess ? FATTN_OK : FATTN_EHIP;
}

int fattn_decode_num_splits(int B, int Hq, int Hkv, int Skv, int d, int num_splits) {
  int st = validate_decode(nullptr, nullptr, nullptr, nullptr, nullptr, nullptr,
                           B, Hq, Hkv, Skv, d, 1.0f, num_splits, false);
  if (st != FATTN_OK) return st;
  int nsplit, chunk;
  plan_splits(B, Hq, Hkv, Skv, num_splits, &nsplit, &chunk);
  return nsplit;
}

size_t fattn_decode_workspace_size(int B, int Hq, int Hkv, int Skv, int d, int num_splits) {
  int nsplit = fattn_decode_num_splits(B, Hq, Hkv, Skv, d, num_splits);
  if (nsplit < 1) return 0;
  return workspace_bytes_for(B, Hq, nsplit, d);
}

int fattn_decode_int8(const void* q, const int8_t* kq, const float* k_scale,
                      const int8_t* vq, const float* v_scale, void* o, float* lse,
                      int B, int Hq, int Hkv, int Skv, int d, float scale,
                      int num_splits, void* workspace, size_t workspace_bytes,
                      void* stream) {
  return decode(q, kq, k_scale, vq, v_scale, o, lse, B, Hq, Hkv, Skv, d, scale, num_splits,
                workspace, workspace_bytes, stream, 8);
}

int fattn_decode_int8_noalloc(const void* q, const int8_t* kq, const float* k_scale,
                              const int8_t* vq, const float* v_scale, void* o, float* lse,
                              int B, int Hq, int Hkv, int Skv, int d, float scale,
                              int num_splits, void* stream) {
  return decode(q, kq, k_scale, vq, v_scale, o, lse, B, Hq, Hkv, Skv, d, scale, num_splits,
                kBuiltinScratch, 0, stream, 8);
}

int fattn_decode_int4(const void* q, const uint8_t* kq, const float* k_scale,
                      const uint8_t* vq, const float* v_scale, void* o, float* lse,
                      int B, int Hq, int Hkv, int Skv, int d, float scale,
                      int num_splits, void* workspace, size_t workspace_bytes,
                      void* stream) {
  return decode(q, kq, k_scale, vq, v_scale, o, lse, B, Hq, Hkv, Skv, d, scale, num_splits,
                workspace, workspace_bytes, stream, 4);
}

int fattn_decode_int8_varlen(const void* q, const int8_t* kq, const float* k_scale,
                             const int8_t* vq, const float* v_scale, const int* seqlens, void* o,
                             float* lse, int B, int Hq, int Hkv, int Skv, int d, float scale,
                             int num_splits, void* workspace, size_t workspace_bytes,
                             void* stream) {
  return decode(q, kq, k_scale, vq, v_scale, o, lse, B, Hq, Hkv, Skv, d, scale, num_splits,
                workspace, workspace_bytes, stream, 8, seqlens, true);
}

int fattn_decode_int4_varlen(const void* q, const uint8_t* kq, const float* k_scale,
                             const uint8_t* vq, const float* v_scale, const int* seqlens, void* o,
                             float* lse, int B, int Hq, int Hkv, int Skv, int d, float scale,
                             int num_splits, void* workspace, size_t workspace_bytes,
                             void* stream) {
  return decode(q, kq, k_scale, vq, v_scale, o, lse, B, Hq, Hkv, Skv, d, scale, num_splits,
                workspace, workspace_bytes, stream, 4, seqlens, true);
}

int fattn_kv_append_int8(const void* x, int8_t* codes, float* scales,
                         int B, int T, int Hkv, int d, int pos, int cap, int dtype, void* stream) {
  return kv_append(x, codes, scales, B, T, Hkv, d, pos, cap, dtype, stream, 8);
}

int fattn_kv_append_int4(const void* x, uint8_t* codes, float* scales,
                         int B, int T, int Hkv, int d, int pos, int cap, int dtype, void* stream) {
  return kv_append(x, codes, scales, B, T, Hkv, d, pos, cap, dtype, stream, 4);
}

const char* fattn_status_string(int status) {
  switch (status) {
    case FATTN_OK: return "ok";
    case FATTN_EINVAL: return "invalid argument";
    case FATTN_EUNSUPPORTED: return "unsupported head_dim or dtype";
    case FATTN_EWORKSPACE: return "workspace missing or too small";
    case FATTN_EHIP: return "HIP kernel launch failed";
    default: return "unknown status";
  }
}

int fattn_version(void) { return kVersion; }

}  // extern "C"
