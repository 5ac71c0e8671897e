/*
 * libfattn -- tiled exact attention for AMD Instinct MI355X (gfx950).
 *
 * C ABI.  Every pointer argument is a DEVICE pointer (memory the caller got
 * from hipMalloc or a framework allocator on the current HIP device) unless
 * stated otherwise; all tensors are dense, row-major and contiguous.  The
 * library allocates and frees nothing, keeps no pointer after a call returns
 * and holds no per-call state, so calls may be issued from several host
 * threads at once.  Work is enqueued asynchronously on `stream` (a
 * hipStream_t passed as void*; NULL is the null stream): buffers must stay
 * alive until that stream has finished the work.  A call makes no HIP call
 * other than its kernel launches on `stream` (no allocation, memset, copy or
 * synchronisation), so calls may be captured into a HIP graph; scalar
 * arguments (sizes, scale, pos, num_splits) are then fixed at capture, while
 * device data such as the varlen lengths is read at each replay.
 *
 * Every device pointer must be 16-byte aligned (allocator-returned pointers
 * are), except cu_seqlens_q/k, seqlens and the lse of fattn_fwd_varlen,
 * which need 4 bytes; a misaligned pointer is rejected with FATTN_EINVAL.
 *
 * Errors: arguments are validated before any HIP call is made.  On any
 * FATTN_E* status except FATTN_EHIP nothing has been enqueued and no output
 * has been written.  FATTN_EHIP means that the HIP runtime refused one of
 * this call's own kernel launches (the status that launch returned); the
 * launches after it were not enqueued.  The library never calls
 * hipGetLastError: an error left pending by the caller's earlier HIP calls
 * is not reported by, and not cleared by, a libfattn call.
 *
 * Sources, cited by page title and section:
 *  [FA-NPU]      "When Transformer meets the Ascend NPU: the memory-slimming
 *                secret of the FlashAttention operator" (ai6s.net/6a0d479d...)
 *  [FA-3MOVES]   the ai6s.net article on FlashAttention's three moves and CANN
 *                8.0 -> 8.5 (ai6s.net/6a0d6a93...)
 *  [FA-VARIANTS] "The FlashAttention variant family: GQA, MQA and sparse
 *                attention, how to choose" (ai6s.net/6a17bd37...)
 */
#ifndef FATTN_H
#define FATTN_H

#include <stddef.h>
#include <stdint.h>

#if defined(__GNUC__) || defined(__clang__)
#define FATTN_API __attribute__((visibility("default")))
#else
#define FATTN_API
#endif

#ifdef __cplusplus
extern "C" {
#endif

/* Status codes returned by every call that can fail. */
typedef enum {
  FATTN_OK = 0,
  FATTN_EINVAL = -1,      /* a NULL or misaligned pointer, a size < 1,
                             Hq % Hkv != 0, an append past the cache end, a
                             non-finite scale, causal not 0/1, window < 0,
                             window > 0 without causal, num_splits < 0, or a
                             tensor too large to index (the prefill and
                             backward also need Hq*d < 2^24 and Hkv*d
                             < 2^25: 32-bit offsets inside a tile) */
  FATTN_EUNSUPPORTED = -2, /* head_dim or dtype outside what the kernels cover */
  FATTN_EWORKSPACE = -3,  /* workspace NULL or smaller than the size query */
  FATTN_EHIP = -4         /* the HIP runtime refused a kernel launch */
} fattn_status;

/* Element type of q, k, v and o in fattn_fwd. */
typedef enum {
  FATTN_F32 = 0, /* float32 in and out, fp32 arithmetic */
  FATTN_BF16 = 1 /* bfloat16 in and out, bf16 matrix products with fp32
                    accumulation and an fp32 softmax */
} fattn_dtype;

/*
 * Exact attention forward (prefill):
 *   o = softmax(scale * q k^T + mask) v,
 * the definition in [FA-NPU] (section on why attention is so memory-hungry)
 * computed tile by tile with an online softmax ([FA-NPU] tiling section;
 * [FA-3MOVES] moves 1 and 2): each query tile streams key/value tiles, keeps
 * per row a running maximum used as the exponent reference and a running sum,
 * rescales its accumulator when the reference rises, and never writes the
 * Sq x Skv score matrix to memory.  The reference is raised lazily (only when
 * a tile's probabilities would exceed 2^8), which leaves the softmax unchanged.
 *
 * q    [B, Sq, Hq, d]   (batch, sequence, heads, head_dim: the order of the
 *                        usage section of [FA-NPU])
 * k, v [B, Skv, Hkv, d]
 * o    [B, Sq, Hq, d]   output, same shape and dtype as q
 * lse  [B, Hq, Sq] fp32 output or NULL: natural log of the row's sum of
 *      exp(scale * q.k) over visible keys (the row statistic the backward
 *      pass recomputes from, [FA-NPU] recomputation section); -inf for a row
 *      with no visible key (its o row is then 0).
 * Hq must be a multiple of Hkv; query head h reads kv head h / (Hq/Hkv), the
 *      head sharing of GQA/MQA ([FA-VARIANTS] GQA section), done in the
 *      kernel without copying k or v.
 * scale: any finite value (1/sqrt(d) in the pages' examples).
 * causal: 0 or 1.  With causal = 1 key j is visible to query i iff
 *      j <= i + (Skv - Sq) (aligned to the last query; the pages' examples
 *      have Sq = Skv, where this is the usual lower triangle).
 * window: 0 = none; W > 0 (needs causal = 1) keeps the W keys
 *      i + (Skv - Sq) - W < j <= i + (Skv - Sq), the query's own position
 *      included ([FA-VARIANTS] local window attention section).
 * d: 64 or 128.  dtype: a fattn_dtype.
 */
FATTN_API int fattn_fwd(const void* q, const void* k, const void* v, void* o, float* lse,
              int B, int Hq, int Hkv, int Sq, int Skv, int d,
              float scale, int causal, int window, int dtype, void* stream);

/*
 * Exact attention over a packed batch of sequences of different lengths (the
 * variable-length batches [FA-3MOVES] lists among CANN's features; the packed
 * layout with cumulative offsets is the library's).  Sequence b owns query
 * rows cu_seqlens_q[b] .. cu_seqlens_q[b+1]-1 and key/value rows
 * cu_seqlens_k[b] .. cu_seqlens_k[b+1]-1 and attends only within itself;
 * causal and window are those of fattn_fwd applied to each sequence's own
 * lengths (Sq_b, Skv_b), so the causal diagonal ends at its last key.  A
 * sequence with no keys gets o = 0 and lse = -inf.
 *
 * q, o   [total_q, Hq, d];  k, v [total_k, Hkv, d]   (dtype as in fattn_fwd)
 * lse    [Hq, total_q] fp32 (natural log) or NULL
 * cu_seqlens_q, cu_seqlens_k  [B+1] int32 device arrays, non-decreasing from
 *        0 to total_q / total_k.  They live on the device and are not checked
 *        on the host: offsets out of range are clamped into the tensors (the
 *        kernels never address outside them) but give unspecified results.
 * max_seqlen_q  the longest Sq_b; it sizes the grid; <= total_q.  If a
 *        sequence is longer, its rows at positions >= max_seqlen_q may be
 *        left unwritten; every row that is written is exact for the
 *        sequence's true lengths (its causal diagonal still ends at its
 *        last key).
 * total_q = 0 is a valid empty call.  Other rules and errors as fattn_fwd.
 */
FATTN_API int fattn_fwd_varlen(const void* q, const void* k, const void* v, void* o, float* lse,
                     const int* cu_seqlens_q, const int* cu_seqlens_k,
                     int B, int Hq, int Hkv, int total_q, int total_k, int max_seqlen_q,
                     int d, float scale, int causal, int window, int dtype, void* stream);

/*
 * Backward pass of fattn_fwd (bf16): the gradients dq, dk, dv of the
 * attention output for an upstream gradient dout, by recomputation ([FA-NPU]
 * recomputation section: the weights are recomputed from the row statistic
 * the forward saved, lse, instead of being stored).  With P the forward's
 * probabilities, D = rowsum(dout * o):
 *   dv = P^T dout,  dS = P * (dout v^T - D),  dq = scale dS k,  dk = scale dS^T q;
 * dk and dv of a kv head sum over the query heads sharing it (GQA / MQA).
 *
 * q, o, dout, dq  [B, Sq, Hq, d] bf16;  k, v, dk, dv  [B, Skv, Hkv, d] bf16
 * lse        [B, Hq, Sq] fp32: the forward's lse for the same q, k, v, scale,
 *            causal and window (o likewise its output)
 * workspace  device scratch of at least fattn_bwd_workspace_size(B, Hq, Hkv,
 *            Sq, Skv, d) bytes; contents on entry do not matter, undefined on
 *            return; concurrent calls need separate workspaces
 * dtype      FATTN_BF16 only (FATTN_F32 returns FATTN_EUNSUPPORTED)
 * Other rules and errors as fattn_fwd; FATTN_EWORKSPACE if the workspace is
 * missing, misaligned or too small.  The result does not depend on
 * scheduling (no atomics): repeated calls give identical bits.
 */
FATTN_API int fattn_bwd(const void* q, const void* k, const void* v, const void* o, const float* lse,
              const void* dout, void* dq, void* dk, void* dv,
              int B, int Hq, int Hkv, int Sq, int Skv, int d,
              float scale, int causal, int window, int dtype,
              void* workspace, size_t workspace_bytes, void* stream);

/* Workspace bytes fattn_bwd needs, 0 if the arguments are invalid: two fp32
 * [B, Hq, Sq] row statistics and, when the query heads of a kv head are split
 * across blocks (few kv heads, many query heads), fp32 partial dk and dv of
 * [splits, B, Skv, Hkv, d] each; every part rounded up to 256 bytes.  Host
 * only; a pure function of its arguments. */
FATTN_API size_t fattn_bwd_workspace_size(int B, int Hq, int Hkv, int Sq, int Skv, int d);

/*
 * Decode over an int8 KV cache ([FA-3MOVES] move 3: the cache stays
 * compressed and is used as is).  One new query token per sequence attends
 * to all Skv cached tokens.  The cache holds per (token, kv head) an int8 row
 * of d codes and one fp32 scale; the key/value the attention sees is
 * code * scale.  The kernel reads the codes from HBM and converts them in
 * registers, folding the scales into the scores and the probabilities.
 * The keys are cut into splits processed in parallel, each producing a
 * partial (o_s, lse_s), and the partials are merged by log-sum-exp (the
 * local-max-and-sum correction of the [FA-NPU] tiling section applied across
 * splits).  With at most 8 splits the splits of a (b, kv head) stream share
 * one workgroup, which merges them on chip: one kernel launch, and the
 * workspace is not touched.  With more, the partials go to the workspace and
 * a second kernel merges them.  With a single split the output is written
 * directly.  Every form gives the same bits for the same split count.
 *
 * q          [B, Hq, d] bf16          (the [B, 1, Hq, d] query of the new token)
 * kq, vq     [B, Hkv, Skv, d] int8    (head-major cache: one contiguous stream
 *                                      per (b, kv head))
 * k_scale, v_scale [B, Hkv, Skv] fp32
 * o          [B, Hq, d] bf16 output;  lse [B, Hq] fp32 output or NULL
 * num_splits 0 = automatic; otherwise the requested number of key splits per
 *            (b, kv head) (the library may use fewer so that none is empty)
 * workspace  device scratch of at least fattn_decode_workspace_size(...)
 *            bytes for the same arguments; its contents on entry do not matter
 *            and on return are undefined.  Concurrent calls need separate
 *            workspaces.
 * d: 64 or 128.  Hq % Hkv == 0.
 */
FATTN_API int fattn_decode_int8(const void* q, const int8_t* kq, const float* k_scale,
                      const int8_t* vq, const float* v_scale, void* o, float* lse,
                      int B, int Hq, int Hkv, int Skv, int d, float scale,
                      int num_splits, void* workspace, size_t workspace_bytes,
                      void* stream);

/*
 * fattn_decode_int8 for callers that cannot allocate device memory: code
 * under HIP graph capture, tight serving loops and harnesses that forbid
 * hipMalloc.  Same operation, arguments (without the workspace), split plan
 * and results, bit for bit.  Plans that merge through partials (more than 8
 * splits per (b, kv head) stream) keep them in a scratch array built into the
 * library instead of a caller workspace: 32 MiB per GPU, allocated when the
 * library's code is loaded on that GPU and held until the process ends; with
 * at most 8 splits nothing beyond o and lse is touched.  Besides its kernel
 * launches the call asks which GPU runs the stream (hipStreamGetDevice, or
 * hipGetDevice for the null stream) and, on its first use of that GPU, takes
 * the array's address there (hipGetSymbolAddress, with the GPU made current
 * for that call and the caller's current device restored); it allocates
 * nothing.  Every call on one GPU shares
 * that GPU's scratch, which keeps the last call's contents (nothing in it has
 * to start at zero): calls that use it and overlap on one GPU (other streams,
 * other host threads) race and must be serialised by the caller.
 *
 * Errors as fattn_decode_int8, plus FATTN_EWORKSPACE when the plan's partials
 * (fattn_decode_workspace_size for the same arguments) exceed the 32 MiB, and
 * FATTN_EHIP when the scratch address cannot be obtained on the stream's GPU.
 */
FATTN_API int fattn_decode_int8_noalloc(const void* q, const int8_t* kq, const float* k_scale,
                      const int8_t* vq, const float* v_scale, void* o, float* lse,
                      int B, int Hq, int Hkv, int Skv, int d, float scale,
                      int num_splits, void* stream);

/*
 * Decode over an int4 KV cache: the same operation, arguments, split plan,
 * workspace size and error behaviour as fattn_decode_int8, with the cache
 * compressed one step further ([FA-3MOVES] move 3 taken to 4-bit codes; the
 * pages give no packing, this is the library's format):
 *
 * kq, vq     [B, Hkv, Skv, d/2] bytes: element 2i of a row is the low nibble
 *            of byte i, element 2i+1 the high nibble, each a signed 4-bit
 *            two's complement code (-8 .. 7; fattn_kv_append_int4 writes
 *            -7 .. 7); the value attention sees is code * scale.
 * k_scale, v_scale [B, Hkv, Skv] fp32, one scale per (token, kv head).
 */
FATTN_API int fattn_decode_int4(const void* q, const uint8_t* kq, const float* k_scale,
                      const uint8_t* vq, const float* v_scale, void* o, float* lse,
                      int B, int Hq, int Hkv, int Skv, int d, float scale,
                      int num_splits, void* workspace, size_t workspace_bytes,
                      void* stream);

/*
 * Decode over a cache whose sequences hold different numbers of tokens (a
 * variable-length batch, [FA-3MOVES] CANN feature list): as
 * fattn_decode_int8 / fattn_decode_int4, with sequence b attending to its
 * first seqlens[b] cached tokens only.  Skv is the cache capacity (the
 * tensors' token dimension); the number of splits and the workspace size
 * are those of the capacity (fattn_decode_num_splits / _workspace_size with
 * Skv), and sequence b's tokens are cut into that many splits of
 * ceil(seqlens[b] / splits) tokens rounded up to a multiple of 64 (splits
 * past its end are empty).
 *
 * seqlens  [B] int32 device array, 0 <= seqlens[b] <= Skv; not checked on the
 *          host (values outside are clamped into [0, Skv]).  A sequence with
 *          0 tokens gets o = 0 and lse = -inf.
 */
FATTN_API int fattn_decode_int8_varlen(const void* q, const int8_t* kq, const float* k_scale,
                      const int8_t* vq, const float* v_scale, const int* seqlens, void* o,
                      float* lse, int B, int Hq, int Hkv, int Skv, int d, float scale,
                      int num_splits, void* workspace, size_t workspace_bytes, void* stream);
FATTN_API int fattn_decode_int4_varlen(const void* q, const uint8_t* kq, const float* k_scale,
                      const uint8_t* vq, const float* v_scale, const int* seqlens, void* o,
                      float* lse, int B, int Hq, int Hkv, int Skv, int d, float scale,
                      int num_splits, void* workspace, size_t workspace_bytes, void* stream);

/*
 * Appends T new tokens to an int8 KV cache (the step that fills the cache
 * fattn_decode_int8 reads; [FA-3MOVES] move 3 names the int8 cache).  For each
 * (b, t, kv head) row x of d values: scale = absmax(x) / 127 in fp32 and
 * code_c = clamp(round-half-even(x_c / scale), -127, 127), with IEEE fp32
 * correctly rounded divisions; an all-zero row gets scale 0 and zero codes.
 *
 * x      [B, T, Hkv, d] (the new tokens' K or V in the prefill layout),
 *        float32 or bfloat16 as dtype says
 * codes  [B, Hkv, cap, d] int8 cache, scales [B, Hkv, cap] fp32: positions
 *        pos .. pos+T-1 of every (b, kv head) stream are written, nothing else
 * Requires 0 <= pos and pos + T <= cap.  d: 64 or 128.  x must be finite
 * (non-finite values give unspecified codes, never a fault).
 */
FATTN_API int fattn_kv_append_int8(const void* x, int8_t* codes, float* scales,
                                   int B, int T, int Hkv, int d, int pos, int cap,
                                   int dtype, void* stream);

/*
 * Appends T new tokens to an int4 KV cache (the cache fattn_decode_int4
 * reads): as fattn_kv_append_int8 with scale = absmax(x) / 7 and codes
 * clamp(round-half-even(x_c / scale), -7, 7), packed two per byte (element
 * 2i in the low nibble of byte i).
 *
 * codes  [B, Hkv, cap, d/2] bytes, scales [B, Hkv, cap] fp32.  Same argument
 *        rules and errors as fattn_kv_append_int8.
 */
FATTN_API int fattn_kv_append_int4(const void* x, uint8_t* codes, float* scales,
                                   int B, int T, int Hkv, int d, int pos, int cap,
                                   int dtype, void* stream);

/* Number of key splits fattn_decode_int8 and fattn_decode_int4 will use for these arguments
 * (>= 1), or a negative fattn_status if they are invalid.  Host only. */
FATTN_API int fattn_decode_num_splits(int B, int Hq, int Hkv, int Skv, int d, int num_splits);

/* Workspace bytes fattn_decode_int8 / fattn_decode_int4 need for these arguments, 0 if they are
 * invalid.  Host only; pure function of its arguments. */
FATTN_API size_t fattn_decode_workspace_size(int B, int Hq, int Hkv, int Skv, int d, int num_splits);

/* Static, NUL-terminated description of a status code.  Host only. */
FATTN_API const char* fattn_status_string(int status);

/* Library version as major * 10000 + minor * 100 + patch.  Host only. */
FATTN_API int fattn_version(void);

#ifdef __cplusplus
}
#endif

#endif /* FATTN_H */
