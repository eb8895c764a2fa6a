/*
 * varlen_attn.h -- C ABI of the MI355X (gfx950) packed variable-length
 * scaled-dot-product attention library (libvarlen_attn.so).
 *
 * Source pages (crate onnx-runtime-ep-cuda, docs.rs source view):
 *   [PVA] src/kernels/packed_varlen_attention.rs, 0.1.0-dev.6
 *   [STD] src/kernels/standard_attention.rs, latest page
 *   [GQA] src/kernels/group_query_attention.rs, latest page
 *
 * What the library computes ([PVA] module doc "Packed layout & cumulative
 * offsets", "Schema (v1)", "Causal alignment"; [STD] module doc "Semantics"):
 * B sequences are concatenated on one token axis. Sequence b owns query rows
 * [cu_seqlens_q[b], cu_seqlens_q[b+1]) and key/value rows
 * [cu_seqlens_kv[b], cu_seqlens_kv[b+1]); nothing attends across sequences.
 * For query head h the kv head is h / (num_heads / kv_num_heads). Scores are
 * scale * (q . k) (the pages fold sqrt(scale) into each operand; that is the
 * same number), then softcap * tanh(s / softcap) when softcap != 0, then the
 * tail-aligned causal mask (query i sees key j iff j <= i + L_kv - L_q), then
 * a stable softmax over the visible keys; a row that sees no key is all
 * zeros. out = softmax . V, accumulated in fp32, stored in the I/O type with
 * round-to-nearest-even.
 *
 * Conventions shared by every entry point:
 *  - Device pointers are HIP device addresses on the current device; host
 *    pointers are ordinary host memory. The library never takes ownership of
 *    a caller's buffer.
 *  - Every argument is validated on the host before any device work is
 *    enqueued; on failure nothing is launched, `out` is untouched, a status
 *    other than VARLEN_OK is returned, and varlen_attn_last_error() holds a
 *    message that begins "varlen_attn_fwd: " (in the spirit of the pages'
 *    op-prefixed KernelFailed errors, [PVA] error helper and execute()).
 *  - Work is enqueued on `stream` (a hipStream_t passed as void*; NULL is the
 *    null stream) and the call returns without synchronizing, except for the
 *    one case documented at varlen_attn_fwd.
 */
#ifndef VARLEN_ATTN_H_
#define VARLEN_ATTN_H_

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* Storage type of Q, K, V and out ([PVA] "Schema (v1)": f32, f16 or bf16,
 * the same for all four). */
typedef enum {
  VARLEN_F32 = 0,
  VARLEN_F16 = 1,
  VARLEN_BF16 = 2
} varlen_dtype_t;

typedef enum {
  VARLEN_OK = 0,
  /* null pointer, num_heads <= 0, kv_num_heads does not divide num_heads,
   * head_dim <= 0, negative or non-finite scale, non-finite softcap, bad
   * dtype code, total_q/total_kv out of range, bf16/f16 q, k, v or out not
   * 16-byte aligned */
  VARLEN_ERR_INVALID_ARGUMENT = 1,
  /* batch < 1, cu[0] != 0, a decreasing cu array, cu[batch] != total
   * ([PVA] execute(): cumulative-array validation) */
  VARLEN_ERR_BAD_SEQLENS = 2,
  /* a dtype / head_dim combination that has no GPU kernel */
  VARLEN_ERR_UNSUPPORTED = 3,
  /* a HIP runtime error (the message carries hipGetErrorString) */
  VARLEN_ERR_DEVICE = 4,
  VARLEN_ERR_OUT_OF_MEMORY = 5
} varlen_status_t;

/*
 * varlen_attn_fwd -- packed varlen attention forward ([PVA] the op's
 * execute(); numerics [PVA] "Numerics & determinism").
 *
 *  q              device, contiguous [total_q, num_heads, head_dim]
 *                 (a [total_q, num_heads*head_dim] tensor has the same bytes)
 *  k              device, contiguous [total_kv, kv_num_heads, head_dim]
 *  v              device, contiguous [total_kv, kv_num_heads, v_head_dim]
 *  cu_seqlens_q   device int32 [batch+1]; may be NULL when the host mirror
 *                 is given
 *  cu_seqlens_kv  device int32 [batch+1]; may be NULL when the host mirror
 *                 is given
 *  cu_seqlens_q_host, cu_seqlens_kv_host
 *                 optional host mirrors of the same arrays. When both are
 *                 given the device arrays are not read at all. When either
 *                 is NULL the library copies the device arrays to the host
 *                 on `stream` and waits for that stream (the only
 *                 synchronizing case, as the pages' op reads cu_seqlens back
 *                 before it launches: [PVA] read_cu_seqlens).
 *  batch          B >= 1
 *  total_q        packed query tokens (rows of q and out), 0 allowed
 *  total_kv       packed key/value tokens
 *  num_heads      Hq >= 1
 *  kv_num_heads   Hkv; <= 0 means Hkv = Hq; must divide Hq
 *  head_dim       D of q and k
 *  v_head_dim     Dv of v and out; <= 0 means Dv = D
 *  dtype          varlen_dtype_t of q, k, v and out
 *  scale          0 selects 1/sqrt(head_dim); otherwise > 0 and finite
 *  is_causal      0 or non-zero (tail-aligned causal mask)
 *  softcap        0 disables; any other finite value c applies
 *                 c * tanh(s / c) (c and -c give the same function)
 *  out            device, caller-allocated [total_q, num_heads, v_head_dim]
 *                 of dtype; every element is written
 *  stream         hipStream_t as void*
 *
 * GPU kernels exist for: bf16 and f16 with head_dim and v_head_dim each in
 * {64, 128} (the two may differ); f32 with head_dim, v_head_dim <= 128.
 * Anything else returns VARLEN_ERR_UNSUPPORTED. With bf16 and f16, q, k, v
 * and out must be 16-byte aligned (the kernels move 16-byte pieces);
 * otherwise the call returns VARLEN_ERR_INVALID_ARGUMENT, after the other
 * checks and before any launch (a call with total_q == 0 is not checked).
 * varlen_attn_fwd_device and varlen_attn_fwd_kvcache apply the same rule.
 *
 * Buffers q, k, v, the cu arrays and out are borrowed and must stay valid
 * until the enqueued work completes. The library keeps a grow-only
 * per-device workspace (work lists, split-KV partials) and serialises calls
 * that use it: a call on another stream waits (on the device) for the
 * previous call's kernels. Results are deterministic run to run: no
 * floating-point atomics, fixed reduction orders.
 */
varlen_status_t varlen_attn_fwd(const void* q, const void* k, const void* v,
                                const int32_t* cu_seqlens_q, const int32_t* cu_seqlens_kv,
                                const int32_t* cu_seqlens_q_host,
                                const int32_t* cu_seqlens_kv_host, int32_t batch,
                                int64_t total_q, int64_t total_kv, int32_t num_heads,
                                int32_t kv_num_heads, int32_t head_dim, int32_t v_head_dim,
                                int32_t dtype, float scale, int32_t is_causal, float softcap,
                                void* out, void* stream);

/*
 * Extra arguments of varlen_attn_fwd_ex. Passing NULL (or a zeroed struct)
 * is the same as varlen_attn_fwd.
 *
 *  local_window   the one field that changes the result: W > 0 keeps, for
 *                 query row i of a sequence, only the keys
 *                 j >= i + L_kv - L_q + 1 - W (the W keys that end at the
 *                 row's tail-aligned diagonal), with or without is_causal
 *                 (page src/kernels/attention.rs, softmax kernel source,
 *                 local_min; page src/kernels/group_query_attention.rs,
 *                 attribute local_window_size). 0 and -1 mean no window
 *                 (-1 is that attribute's default; 0 is what a zeroed struct
 *                 holds); below -1 returns VARLEN_ERR_INVALID_ARGUMENT.
 *
 * The other fields steer how the work is split, for tests that prove the
 * paths agree and for tuning; the result is the same for every value of
 * them up to fp32 rounding.
 *
 *  decode_path    0 auto (split-KV decode kernel for sequences with L_q == 1
 *                 on bf16/f16), 1 never (every sequence through the prefill
 *                 kernel), 2 same as auto
 *  decode_chunk   keys per split-KV work item; 0 picks automatically
 *                 (rounded up to a multiple of 128)
 *  prefill_kv_chunk  > 0: keys per prefill work item, long key ranges being
 *                 split across workgroups and recombined by the log-sum-exp
 *                 combine (rounded up to a multiple of 64); 0 or < 0: no
 *                 split, one item covers a row block's whole key range (the
 *                 faster choice on the long-context workload: splitting at
 *                 8192 / 4096 / 2048 keys measured 9 / 22 / 31 % slower)
 */
typedef struct {
  int32_t decode_path;
  int32_t decode_chunk;
  int32_t prefill_kv_chunk;
  int32_t local_window;
  int32_t reserved[4];
} varlen_attn_options_t;

varlen_status_t varlen_attn_fwd_ex(const void* q, const void* k, const void* v,
                                   const int32_t* cu_seqlens_q, const int32_t* cu_seqlens_kv,
                                   const int32_t* cu_seqlens_q_host,
                                   const int32_t* cu_seqlens_kv_host, int32_t batch,
                                   int64_t total_q, int64_t total_kv, int32_t num_heads,
                                   int32_t kv_num_heads, int32_t head_dim, int32_t v_head_dim,
                                   int32_t dtype, float scale, int32_t is_causal,
                                   float softcap, void* out, void* stream,
                                   const varlen_attn_options_t* options);

/*
 * varlen_attn_fwd_device -- the same op for callers that cannot wait for the
 * host: CUDA/HIP-graph capture and replay, or loops that must never stall on
 * a device-to-host read. The packed op of the pages reads cu_seqlens back and
 * synchronises, so it cannot be captured (page
 * src/kernels/packed_varlen_attention.rs, capture_support); this entry point
 * builds the work list on the device instead, validates the cu arrays there
 * and reports violations through an error latch, as the GQA op's capture-safe
 * decode does (page src/kernels/group_query_attention.rs,
 * gqa_prepare_metadata and its capture-error bit flags).
 *
 * The call enqueues a scheduler kernel and the attention kernels on `stream`
 * and returns. It reads no host memory, allocates nothing, copies nothing
 * from the host and never synchronises, so it can be captured into a graph;
 * a replay reads the cu arrays (and q, k, v) as they are at replay time.
 * Usually everything runs on `stream`: the scheduler, the split-KV decode,
 * then the prefill launch, whose last workgroups also merge the decode
 * splits. When total_q <= batch (a decode-dominated batch) the decode and
 * combine kernels run on a library-owned side stream of the device, forked
 * from `stream` after the scheduler and joined back into it before the call
 * returns, so the call keeps the ordering of a single stream. The side
 * stream is created by the first such call outside a graph capture; until
 * then (and inside a capture that comes first) the one-stream form runs.
 *
 *  q, k, v, out   as varlen_attn_fwd
 *  cu_seqlens_q, cu_seqlens_kv
 *                 device int32 [batch + 1], read only on the device
 *  total_q        rows of the q and out buffers; cu_seqlens_q[batch] may be
 *                 any value up to it (rows past it are not written)
 *  total_kv       rows of the k and v buffers; cu_seqlens_kv[batch] <= it
 *  local_window   as the options field of varlen_attn_fwd_ex (-1 or 0: none)
 *  workspace      device memory of at least
 *                 varlen_attn_device_workspace_bytes(...) bytes, 256-byte
 *                 aligned, owned by the caller; a call overwrites it, so
 *                 calls that overlap on the device need separate workspaces
 *  error_latch    device int32, owned by the caller, zero before first use.
 *                 The scheduler ORs a violation into it: 1 cu_seqlens_q[0]
 *                 != 0, 2 cu_seqlens_q decreases, 4 cu_seqlens_q[batch] >
 *                 total_q, 8/16/32 the same for cu_seqlens_kv, 64 internal
 *                 list overflow. While it is non-zero, calls compute nothing
 *                 and leave out untouched; clear it (with a kernel, not a
 *                 memset, inside a graph) to resume.
 *
 * Host-side argument errors return their status before anything is enqueued
 * (the rules of varlen_attn_fwd, on the scalars only). The same GPU kernels
 * as varlen_attn_fwd run on the same items, so the results are bitwise those
 * of varlen_attn_fwd with default options.
 */
size_t varlen_attn_device_workspace_bytes(int32_t batch, int64_t total_q, int64_t total_kv,
                                          int32_t num_heads, int32_t kv_num_heads, int32_t head_dim,
                                          int32_t v_head_dim, int32_t dtype);

varlen_status_t varlen_attn_fwd_device(const void* q, const void* k, const void* v,
                                       const int32_t* cu_seqlens_q, const int32_t* cu_seqlens_kv,
                                       int32_t batch, int64_t total_q, int64_t total_kv,
                                       int32_t num_heads, int32_t kv_num_heads, int32_t head_dim,
                                       int32_t v_head_dim, int32_t dtype, float scale,
                                       int32_t is_causal, float softcap, int32_t local_window,
                                       void* out, void* workspace, size_t workspace_bytes,
                                       int32_t* error_latch, void* stream);

/*
 * varlen_attn_fwd_device_ex -- varlen_attn_fwd_device with the options
 * struct, of which this path takes decode_path: 0 or 2 auto (sequences with
 * L_q == 1 go to the split-KV decode kernel on bf16/f16), 1 never (every
 * sequence through the prefill kernel). With 1 the decode and combine
 * launches are left out, which suits a caller that knows its batches have
 * no single-row sequences (a prefill-only phase); the output is the same
 * softmax up to rounding, and bit-identical to the host-planned call with
 * the same decode_path. decode_chunk and prefill_kv_chunk of the struct
 * must be 0 and its local_window 0 or -1 (the window is the local_window
 * argument), else
 * VARLEN_ERR_INVALID_ARGUMENT; NULL options mean all zero. The workspace
 * size of varlen_attn_device_workspace_bytes covers either decode_path.
 * Every other argument, and the capture rules, as varlen_attn_fwd_device.
 */
varlen_status_t varlen_attn_fwd_device_ex(const void* q, const void* k, const void* v,
                                          const int32_t* cu_seqlens_q, const int32_t* cu_seqlens_kv,
                                          int32_t batch, int64_t total_q, int64_t total_kv,
                                          int32_t num_heads, int32_t kv_num_heads, int32_t head_dim,
                                          int32_t v_head_dim, int32_t dtype, float scale,
                                          int32_t is_causal, float softcap, int32_t local_window,
                                          void* out, void* workspace, size_t workspace_bytes,
                                          int32_t* error_latch, void* stream,
                                          const varlen_attn_options_t* options);

/*
 * varlen_attn_fwd_device_noalloc -- varlen_attn_fwd_device for callers that
 * cannot allocate device memory at all, not even a workspace of their own:
 * code under HIP-graph capture that must not call hipMalloc, tight serving
 * loops, harnesses that forbid allocation. It takes the same arguments
 * without the workspace and behaves like varlen_attn_fwd_device with default
 * options, with the same kernels on the same items (bitwise the same
 * output), always in the one-stream form (no side stream).
 *
 * The work list and split-KV partials live in a static device array of
 * VARLEN_NOALLOC_SCRATCH_BYTES bytes inside the library, of which every GPU
 * the library runs on holds its own copy until the process ends (its device
 * address is looked up on the first such call on a GPU). The call allocates
 * nothing: no hipMalloc, hipFree, stream or event (kernel timing through
 * varlen_attn_profile_enable does not record this call). A batch whose work
 * list needs more than that many bytes (the size varlen_attn_device_workspace_
 * bytes reports, e.g. about 25 MB for 256 decode rows against 4.2 M keys)
 * returns VARLEN_ERR_INVALID_ARGUMENT before anything is enqueued. Every
 * such call on one GPU shares the one array, and each call overwrites it:
 * calls that overlap on a GPU (different streams, threads or captured graphs
 * in flight at once) race and must be serialised by the caller. Nothing in
 * the array needs to be cleared between calls.
 */
#define VARLEN_NOALLOC_SCRATCH_BYTES (32u << 20)

varlen_status_t varlen_attn_fwd_device_noalloc(const void* q, const void* k, const void* v,
                                               const int32_t* cu_seqlens_q, const int32_t* cu_seqlens_kv,
                                               int32_t batch, int64_t total_q, int64_t total_kv,
                                               int32_t num_heads, int32_t kv_num_heads, int32_t head_dim,
                                               int32_t v_head_dim, int32_t dtype, float scale,
                                               int32_t is_causal, float softcap, int32_t local_window,
                                               void* out, int32_t* error_latch, void* stream);

/*
 * varlen_kv_append_rope -- the step before a decode (or chunked-prefill) call
 * over a fixed-capacity KV cache: rotary position embedding of the new query
 * and key rows, and the append of the new key and value rows into the cache,
 * in one launch (page src/kernels/group_query_attention.rs: the rotary kernel
 * gqa_rope_bnsh, the cache kernels gqa_build_cache / gqa_append_cache and the
 * fused single-token prep gqa_fuse_decode_prep; page src/kernels/attention.rs,
 * the fixed-capacity, fixed-slot append test). Capture-safe like
 * varlen_attn_fwd_device: it only enqueues one kernel on `stream`.
 *
 * Rows are packed by cu_seqlens_q as in varlen_attn_fwd. The cache keeps the
 * attention's row format: k_cache [batch * cache_capacity, Hkv, D] and
 * v_cache [batch * cache_capacity, Hkv, Dv], sequence b owning rows
 * [b * cache_capacity, (b + 1) * cache_capacity), of which the first
 * cache_seqlens[b] hold earlier tokens.
 *
 *  q, q_out       device [total_q rows, q_row_stride] new query rows and
 *                 dense [total_q, Hq, D] rotated output; q_out may equal q
 *                 (in place, dense rows only); both NULL: no query work
 *  k, v           device new key / value rows, k_row_stride / v_row_stride
 *                 elements apart (0: dense, Hkv*D and Hkv*Dv). A packed QKV
 *                 buffer [total_q, (Hq + 2 Hkv) * D] is passed as q = base,
 *                 k = base + Hq*D, v = base + (Hq + Hkv)*D with all three
 *                 strides (Hq + 2 Hkv) * D. May be NULL when total_q == 0
 *                 (no new rows: the call only writes kv_seqlens_out)
 *  k_cache, v_cache  device caches as above; new row i of sequence b goes
 *                 to row b * cache_capacity + cache_seqlens[b] + i; no other
 *                 cache row is written
 *  cu_seqlens_q   device int32 [batch + 1]
 *  cache_seqlens  device int32 [batch], tokens already in each sequence
 *  kv_seqlens_out device int32 [batch] or NULL; receives cache_seqlens[b] +
 *                 L_q[b], the key count of the attention call over the cache
 *  cos_cache, sin_cache  device fp32 [rotary_rows, rotary_dim / 2]
 *  position_ids   device int64 [total_q] or NULL; the position of each new
 *                 row (default cache_seqlens[b] + i)
 *  rotary_dim     0: no rotation (a plain append); else even in [2, D]. Pair
 *                 m < rotary_dim/2 of every query and key head is dims
 *                 (2m, 2m+1) if rotary_interleaved, else (m, m +
 *                 rotary_dim/2); it turns by the table angle at the row's
 *                 position: (a, b) -> (a*cos - b*sin, a*sin + b*cos). Dims
 *                 from rotary_dim on are copied. Values are never turned.
 *  dtype          storage type of q, k, v, q_out and the caches; the rotation
 *                 is worked in fp32 and rounded to nearest even
 *  error_latch    as varlen_attn_fwd_device (the same word can serve both
 *                 calls). Bits: 1/2/4 cu_seqlens_q as there, 128
 *                 cache_seqlens[b] < 0, 256 cache_seqlens[b] + L_q[b] >
 *                 cache_capacity, 512 a position outside [0, rotary_rows).
 *                 A row whose sequence or position is invalid writes
 *                 nothing; a workgroup that finds the latch already set
 *                 writes nothing, so after an error the step's outputs are
 *                 unspecified (and the attention call that follows computes
 *                 nothing until the latch is cleared).
 *
 * Requires D and Dv even, batch * cache_capacity < 2^31. Buffers are
 * borrowed; nothing is allocated.
 */
varlen_status_t varlen_kv_append_rope(const void* q, void* q_out, const void* k, const void* v,
                                      int64_t q_row_stride, int64_t k_row_stride, int64_t v_row_stride,
                                      void* k_cache, void* v_cache, const int32_t* cu_seqlens_q,
                                      const int32_t* cache_seqlens, int32_t* kv_seqlens_out,
                                      const float* cos_cache, const float* sin_cache,
                                      const int64_t* position_ids, int32_t batch, int64_t total_q,
                                      int32_t num_heads, int32_t kv_num_heads, int32_t head_dim,
                                      int32_t v_head_dim, int32_t dtype, int32_t cache_capacity,
                                      int32_t rotary_dim, int32_t rotary_rows, int32_t rotary_interleaved,
                                      int32_t* error_latch, void* stream);

/*
 * varlen_attn_fwd_kvcache -- varlen_attn_fwd_device with the keys and values
 * in a fixed-capacity cache instead of packed by cu_seqlens_kv: sequence b
 * attends to cache rows [b * cache_capacity, b * cache_capacity +
 * kv_seqlens[b]) (the attention read is bounded to the valid rows; the rest
 * of the cache is never read, per the fixed-capacity append path of page
 * src/kernels/attention.rs). The causal mask stays tail-aligned: query row i
 * of sequence b sees key j <= i + kv_seqlens[b] - L_q[b].
 *
 *  k_cache, v_cache  device [batch * cache_capacity, Hkv, D] / [..., Dv]
 *  kv_seqlens     device int32 [batch] (e.g. kv_seqlens_out of
 *                 varlen_kv_append_rope); a length < 0 or > cache_capacity
 *                 sets bit 1024 of the latch
 *  workspace      at least varlen_attn_device_workspace_bytes(batch,
 *                 total_q, batch * cache_capacity, ...) bytes
 *
 * Everything else as varlen_attn_fwd_device (bits 8/16/32 are not used).
 */
varlen_status_t varlen_attn_fwd_kvcache(const void* q, const void* k_cache, const void* v_cache,
                                        const int32_t* cu_seqlens_q, const int32_t* kv_seqlens,
                                        int32_t batch, int64_t total_q, int32_t cache_capacity,
                                        int32_t num_heads, int32_t kv_num_heads, int32_t head_dim,
                                        int32_t v_head_dim, int32_t dtype, float scale,
                                        int32_t is_causal, float softcap, int32_t local_window,
                                        void* out, void* workspace, size_t workspace_bytes,
                                        int32_t* error_latch, void* stream);

/*
 * varlen_attn_plan -- the host-side work scheduler on its own (no device
 * work, no HIP call; usable without a GPU). It validates like
 * varlen_attn_fwd (with host cu arrays) and fills `stats` with what a call
 * with these arguments would launch. When `items` is non-NULL and
 * `items_capacity` (in int32 elements) is large enough, it also writes the
 * work items, VARLEN_PLAN_ITEM_INTS int32 each, kernel by kernel in launch
 * order. Each item is:
 *   { kind, seq, q_row_begin, q_rows, head_begin, heads, kv_begin, kv_end,
 *     partial_base, n_splits, q_token0, kv_token0, L_q, L_kv, split, 0 }
 * kind 0 = prefill (MFMA), 1 = prefill (fp32), 2 = split-KV decode,
 * 3 = log-sum-exp combine. q_row_begin and kv_begin/kv_end are local to the
 * sequence, q_token0/kv_token0 are cu_seqlens_q[seq]/cu_seqlens_kv[seq].
 * partial_base is -1 when the item writes `out` directly; otherwise the
 * item (split `split` of `n_splits`) writes fp32 partial rows starting at
 * partial_base, and the combine item with the same partial_base merges the
 * n_splits partials of every (row, head) into `out`.
 * Returns VARLEN_OK or the validation status; VARLEN_ERR_INVALID_ARGUMENT if
 * the item buffer is too small (stats are still filled).
 */
#define VARLEN_PLAN_ITEM_INTS 16
typedef struct {
  int64_t n_prefill_items;
  int64_t n_decode_items;
  int64_t n_combine_items;
  int64_t n_partials;        /* fp32 partial rows (head x D+2 floats each) */
  int64_t valid_pairs;       /* (query row, key) pairs the mask leaves visible */
  int64_t visited_pairs;     /* pairs the scheduled tiles cover (>= valid_pairs) */
  int64_t workspace_bytes;   /* device workspace the call needs */
  int32_t waves_per_prefill_item;
  int32_t heads_per_item;
  int32_t reserved[6];
} varlen_attn_plan_stats_t;

varlen_status_t varlen_attn_plan(const int32_t* cu_seqlens_q_host,
                                 const int32_t* cu_seqlens_kv_host, int32_t batch,
                                 int64_t total_q, int64_t total_kv, int32_t num_heads,
                                 int32_t kv_num_heads, int32_t head_dim, int32_t v_head_dim,
                                 int32_t dtype, float scale, int32_t is_causal, float softcap,
                                 const varlen_attn_options_t* options,
                                 varlen_attn_plan_stats_t* stats, int32_t* items,
                                 int64_t items_capacity);

/*
 * Number of (query row, key) pairs the mask leaves visible for host cu
 * arrays ([PVA] "Causal alignment"): sum over sequences of L_q * L_kv, or
 * with is_causal of sum_i clamp(i + L_kv - L_q + 1, 0, L_kv). Returns -1 on
 * invalid arrays. The attention FLOPs of a call are 2 * pairs * Hq * (D + Dv)
 * (QK^T and P.V, 2 flops per multiply-add).
 */
int64_t varlen_attn_valid_pairs(const int32_t* cu_seqlens_q_host,
                                const int32_t* cu_seqlens_kv_host, int32_t batch,
                                int32_t is_causal);

/* The same count with a local window of local_window keys (<= 0: none): row i
 * sees the keys j in [max(0, i + off + 1 - W), hi), off = L_kv - L_q, hi =
 * clamp(i + off + 1, 0, L_kv) with is_causal and L_kv without. Returns -1 on
 * invalid arrays. */
int64_t varlen_attn_valid_pairs_window(const int32_t* cu_seqlens_q_host,
                                       const int32_t* cu_seqlens_kv_host, int32_t batch,
                                       int32_t is_causal, int32_t local_window);

/*
 * Kernel timing for measurement tools (not needed for computing). While
 * enabled, every call records a pair of HIP events on its stream around each
 * kernel it launches. varlen_attn_profile_read waits for the recorded events,
 * adds their elapsed times to per-kernel totals and returns the totals since
 * the last enable. Index k of the arrays: 0 prefill (MFMA), 1 prefill
 * (fp32), 2 split-KV decode, 3 combine, 4 work-list upload, 5 device
 * scheduler (varlen_attn_fwd_device, varlen_attn_fwd_kvcache), 6 cache step
 * (varlen_kv_append_rope).
 * varlen_attn_profile_enable(0) stops recording; (1) clears and starts.
 */
#define VARLEN_PROFILE_KINDS 7
typedef struct {
  double total_ms[VARLEN_PROFILE_KINDS];
  int64_t launches[VARLEN_PROFILE_KINDS];
  int64_t items[VARLEN_PROFILE_KINDS];  /* workgroups launched (upload: bytes) */
} varlen_attn_profile_t;

varlen_status_t varlen_attn_profile_enable(int32_t enable);
varlen_status_t varlen_attn_profile_read(varlen_attn_profile_t* out);

/* Message of the last failed call on this thread ("" if none). The pointer
 * stays valid until the next call on this thread. */
const char* varlen_attn_last_error(void);

/* Frees the workspace of every device (after waiting for its last use).
 * Safe to call at any time; the next call allocates again. */
varlen_status_t varlen_attn_release(void);

/* Library version as "major.minor.patch". */
const char* varlen_attn_version(void);

#ifdef __cplusplus
}
#endif

#endif /* VARLEN_ATTN_H_ */
