// Internal interface between the C-ABI layer (fattn_api.cpp) and the kernel
// translation units.  Not installed; the public interface is include/fattn.h.
#pragma once

#include <hip/hip_runtime.h>
#include <cstdint>
#include <tuple>

namespace fattn {

// Arguments of one prefill call after validation.  Pointers are device
// pointers; q/o are [B, Sq, Hq, d], k/v [B, Skv, Hkv, d], lse [B, Hq, Sq] or null.
// Packed variable-length batches set cu_q / cu_k ([B+1] device offsets): then
// q/o are [total_q, Hq, d], k/v [total_k, Hkv, d], lse [Hq, total_q], and Sq /
// Skv are the longest sequence lengths (they size the grid).
struct FwdArgs {
  const void* q;
  const void* k;
  const void* v;
  void* o;
  float* lse;
  int B, Hq, Hkv, Sq, Skv, d;
  float scale;
  int causal;
  int window;
  const int* cu_q = nullptr;
  const int* cu_k = nullptr;
  int total_q = 0;
  int total_k = 0;
};

// Arguments of one quantised-cache decode call after validation and split planning.
struct DecodeArgs {
  const void* q;          // [B, Hq, d] bf16
  const void* kq;         // [B, Hkv, Skv, d * bits / 8] codes
  const float* kscale;    // [B, Hkv, Skv]
  const void* vq;
  const float* vscale;
  void* o;                // [B, Hq, d] bf16
  float* lse;             // [B, Hq] or null
  int B, Hq, Hkv, Skv, d;
  float scale;
  int nsplit;             // key splits per (b, kv head)
  int chunk;              // tokens per split (a multiple of the kernel's key tile)
  float* part_o;          // workspace: [B, Hq, nsplit, d] fp32
  float* part_lse;        // workspace: [B, Hq, nsplit] fp32
  int bits;               // code width: 8 (int8) or 4 (two int4 codes per byte)
  const int* seqlens = nullptr;  // [B] device lengths (first seqlens[b] tokens), or null
};

// Arguments of one KV-cache append after validation.
struct KvQuantArgs {
  const void* x;          // [B, T, Hkv, d] bf16 or fp32
  void* codes;            // [B, Hkv, cap, d * bits / 8]
  float* scales;          // [B, Hkv, cap]
  int B, T, Hkv, d, pos, cap;
  bool bf16;
  int bits;               // 8: int8 codes, scale absmax/127; 4: packed int4, absmax/7
};

// Arguments of one backward call after validation (bf16, dense layout).
struct BwdArgs {
  const void* q;          // [B, Sq, Hq, d]
  const void* k;          // [B, Skv, Hkv, d]
  const void* v;
  const void* o;          // forward output [B, Sq, Hq, d]
  const float* lse;       // forward lse [B, Hq, Sq]
  const void* dout;       // upstream gradient [B, Sq, Hq, d]
  void* dq;               // [B, Sq, Hq, d]
  void* dk;               // [B, Skv, Hkv, d]
  void* dv;
  int B, Hq, Hkv, Sq, Skv, d;
  float scale;
  int causal;
  int window;
  float* l2;              // workspace [B, Hq, Sq]
  float* dd;              // workspace [B, Hq, Sq]
  float* part_k;          // workspace [nsplit, B, Skv, Hkv, d] (nsplit > 1 only)
  float* part_v;
};

// Query-head splits of the dK/dV kernel (1: no partials).
int bwd_head_splits(int B, int Hq, int Hkv, int Skv);

hipError_t launch_fwd_f32(const FwdArgs& a, hipStream_t stream);
hipError_t launch_bwd_bf16(const BwdArgs& a, hipStream_t stream);
hipError_t launch_fwd_bf16(const FwdArgs& a, hipStream_t stream);
hipError_t launch_decode(const DecodeArgs& a, hipStream_t stream);
hipError_t launch_kv_quant(const KvQuantArgs& a, hipStream_t stream);

// Key-tile length of the decode split kernel; split chunks are multiples of it.
constexpr int kDecodeTile = 64;

// Most splits per (b, kv head) stream that one workgroup holds and merges on
// chip; plans with more splits merge through the workspace partials.
constexpr int kDecodeWgMaxSplits = 8;

// Size of the decode's built-in scratch array (one per GPU, allocated when the
// library's code object is loaded on that GPU and held until the process
// ends), used instead of a caller workspace by fattn_decode_int8_noalloc.
constexpr size_t kDecodeScratchBytes = size_t(32) << 20;

// Device address of the built-in scratch array on the GPU that runs `stream`
// (hipGetSymbolAddress with that GPU current, taken once per device and kept).
hipError_t decode_scratch(hipStream_t stream, void** ptr);

// Enqueues kernel<<<grid, block, lds, stream>>>(args...) and returns the
// status of that launch itself (hipLaunchKernel's result), never an error
// left pending by an earlier HIP call: the library does not call
// hipGetLastError, so such an error is neither reported nor consumed here.
template <typename... P, typename... A>
hipError_t launch_kernel(void (*kernel)(P...), dim3 grid, dim3 block, size_t lds,
                         hipStream_t stream, A... args) {
  static_assert(sizeof...(P) == sizeof...(A), "argument count");
  auto typed = std::make_tuple(P(args)...);
  void* ptrs[sizeof...(P)];
  std::apply([&](auto&... x) {
    int i = 0;
    ((ptrs[i++] = static_cast<void*>(&x)), ...);
  }, typed);
  return hipLaunchKernel(reinterpret_cast<const void*>(kernel), grid, block, ptrs, lds, stream);
}

}  // namespace fattn
