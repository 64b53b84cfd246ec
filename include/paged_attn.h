/*
 * paged_attn.h -- C ABI of the MI355X (gfx950) paged GQA decode-attention library.
 *
 * The operation (page "Paged Attention Kernel Architecture for BI-V100", section 1
 * "Problem Definition"): for each sequence b and query head h,
 *
 *     out[b,h,:] = softmax_t( scale * q[b,h,:] . K[t,:] ) . V[t,:],   0 <= t < L_b,
 *
 * where L_b = cache_seqlens[b] and token t of sequence b is stored in physical
 * block block_table[b][t / block_size] at offset t % block_size (same page,
 * section 3 "Paged K/V Gather"; the decode-path example of the transformers
 * "Paged attention" docs page, where the table has shape (batch,
 * max_blocks_per_seq) and -1 marks an unassigned entry). Query head h reads KV
 * head h / G, G = num_q_heads / num_kv_heads: G consecutive query heads share one
 * KV head (same page, section 4 "GQA Handling"). One query token per sequence.
 *
 * The work is split into KV partitions of partition_size tokens; each partition
 * keeps a running softmax state (max, sum, unnormalised output) and a second
 * kernel merges the partitions with the max-rescaling combine (same page,
 * section 2 and section 6 "Kernel Launch Configuration"; page
 * "v10_triton_paged_gqa", core principle, for the per-tile update).
 *
 * Conventions for every entry point:
 *   - All array pointers given to paged_attn_decode are DEVICE pointers owned by
 *     the caller; the library never frees or keeps them after the call returns.
 *   - Nothing here allocates device memory. Partial results live in a caller
 *     workspace of paged_attn_workspace_size() bytes (paged_attn_decode_static:
 *     in a static array inside the library).
 *   - Functions return PA_OK (0) or a negative PA_E_* code; on error nothing is
 *     launched and nothing aborts. paged_attn_strerror() names the code.
 *   - Sizes are in elements unless they say bytes.
 */
#ifndef PAGED_ATTN_H
#define PAGED_ATTN_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define PA_ABI_VERSION 5

/* Element type of the K and V caches. q and out are always float32. */
typedef enum pa_dtype { PA_DTYPE_F32 = 0, PA_DTYPE_F16 = 1, PA_DTYPE_BF16 = 2 } pa_dtype;

/* Which partition kernel runs: VALU (vector ALU dot products and reductions) or
 * MFMA (matrix-core micro-GEMMs for the G x d . d x N scores and the P . V
 * product). MFMA needs f16 or bf16 K/V and has two kernels: MFMA_STREAM, a
 * persistent kernel in which each wave streams an equal share of the batch's
 * 16-token chunks (block_size >= 16, batch <= 1024, fewer than 2^31 chunks per
 * KV head: batch * ceil(max_blocks_per_seq * block_size / 16) < 2^31), and
 * MFMA_GRID, one workgroup per partition (any block size and batch).
 * PA_PATH_MFMA picks MFMA_STREAM when it applies and the batch's K/V bound
 * (batch * num_kv_heads * max_blocks_per_seq * block_size * head_dim * 2
 * elements) is at least 160 MB, else MFMA_GRID (on smaller batches the
 * persistent waves' start-up is not amortised); AUTO picks MFMA that way for
 * 16-bit K/V and VALU for fp32.
 *
 * MFMA_FUSED is MFMA_GRID with the partition merge done by the last partition
 * workgroup of each (sequence, KV head) to finish, instead of by a second
 * kernel (the single-launch variant of page "Paged Attention Kernel
 * Architecture for BI-V100", section 2): one launch per call. Its workspace
 * starts with batch * num_kv_heads int32 arrival counters (at offset 0), which
 * must be zero when a call starts; every call leaves them zero, so zero the
 * workspace once after allocating it (or after using it for anything else).
 * Calls that share a workspace must not overlap in time. One wave reads all
 * of a KV head's partition states, so it suits short contexts; it needs
 * 2 * n_part * G + 16 <= 16 * head_dim, n_part = ceil(max_blocks_per_seq *
 * block_size / partition_size) (else PA_E_PARTITION). */
typedef enum pa_path {
  PA_PATH_AUTO = 0,
  PA_PATH_VALU = 1,
  PA_PATH_MFMA = 2,
  PA_PATH_MFMA_GRID = 3,
  PA_PATH_MFMA_STREAM = 4,
  PA_PATH_MFMA_FUSED = 5
} pa_path;

/* Status codes. */
#define PA_OK 0
#define PA_E_NULL (-1)        /* a required pointer is NULL                          */
#define PA_E_SHAPE (-2)       /* sizes <= 0, batch or num_q_heads > 65535,           */
                              /* num_q_heads % num_kv_heads != 0, or G beyond what   */
                              /* the selected path supports (VALU: G <= 8, MFMA:     */
                              /* G <= 16)                                            */
#define PA_E_HEAD_DIM (-3)    /* head_dim not 64, 128 or 256                         */
#define PA_E_BLOCK_SIZE (-4)  /* block_size not a power of two in [1, 1024]          */
#define PA_E_DTYPE (-5)       /* kv_dtype not a pa_dtype                             */
#define PA_E_STRIDE (-6)      /* a stride <= 0, token stride < head_dim, or a stride */
                              /* that is not a multiple of 16 bytes (with            */
                              /* PA_FLAG_KV_XPACKED: token strides not x and 1, or a */
                              /* head stride < block_size * head_dim)                */
#define PA_E_ALIGN (-7)       /* q, out, k_cache or v_cache not 16-byte aligned      */
#define PA_E_PARTITION (-8)   /* partition_size not 0 and not a multiple of 32 in    */
                              /* [32, 16384], or spanning more than 1024 blocks, or  */
                              /* (MFMA_FUSED) 2 * n_part * G + 16 > 16 * head_dim    */
#define PA_E_WORKSPACE (-9)   /* workspace NULL or smaller than required             */
#define PA_E_PATH (-10)       /* path not a pa_path, an MFMA path asked for f32 K/V, */
                              /* or MFMA_STREAM asked for block_size < 16, batch     */
                              /* > 1024 or 2^31 chunks or more                       */
#define PA_E_LAUNCH (-11)     /* the HIP runtime refused a launch                    */
#define PA_E_TABLE (-12)      /* (check_inputs) an entry read for an attended token  */
                              /* is outside [0, num_blocks)                           */
#define PA_E_SEQLEN (-13)     /* (check_inputs) a cache length < 0 or > MBS * bs     */
#define PA_E_NOMEM (-14)      /* (block manager) not enough free blocks              */
#define PA_E_SEQ (-15)        /* (block manager) unknown sequence, index or length   */
#define PA_E_SCRATCH (-16)    /* (paged_attn_decode_static) the call needs more      */
                              /* workspace than PA_STATIC_SCRATCH_BYTES               */

/* pa_desc.flags bits. */
#define PA_FLAG_KV_SHARED 1  /* physical blocks may be listed by several sequences   */
                             /* (prefix sharing, as the block manager of the        */
                             /* paged-attention-runtime design notes does): K/V     */
                             /* loads stay cacheable (without the flag they are     */
                             /* non-temporal), and on the streaming path sequences  */
                             /* are taken in groups of F = 16 / G (G <= 8): the     */
                             /* leading blocks that all of a group's members list   */
                             /* (the same valid block ids) and attend whole, at     */
                             /* least 256 tokens, are read once for the group, its  */
                             /* F x G query heads filling the score MFMA's 16       */
                             /* columns; each member's remaining tokens are its own */
                             /* stream, and the combine merges the two. Results do  */
                             /* not depend on the grouping beyond rounding. Members */
                             /* of one family are best adjacent in the batch.       */
#define PA_FLAG_QO_BF16 2    /* q and out are bf16 instead of fp32 (accumulation,     */
                             /* partial states and the combine stay fp32; out is      */
                             /* rounded to nearest even once, at the end)             */
#define PA_FLAG_KV_XPACKED 4 /* the cache layout of page "Paged Attention Kernel      */
                             /* Architecture for BI-V100", section 3: K is            */
                             /* [num_blocks, num_kv_heads, d/x, block_size, x] with   */
                             /* x = 16 bytes / element size, V is                     */
                             /* [num_blocks, num_kv_heads, d, block_size]. Block and  */
                             /* head strides come from the descriptor; each (block,   */
                             /* head) tile is dense, so k_stride_token must be x and  */
                             /* v_stride_token 1, and head strides >= block_size * d. */
                             /* f16/bf16 K/V and block_size >= 8 only. Decode runs on */
                             /* MFMA_GRID or MFMA_FUSED (AUTO and MFMA pick           */
                             /* MFMA_GRID); VALU, MFMA_STREAM and paged_attn_prefill  */
                             /* return PA_E_PATH. Append and copy_blocks accept it.   */

/* Bits the kernels OR into the optional device status word. */
#define PA_STATUS_BAD_BLOCK 1   /* an attended token's table entry was outside [0, NB) */
                                /* (that token was skipped, never dereferenced)        */
#define PA_STATUS_BAD_SEQLEN 2  /* a cache length was < 0 or > MBS * bs (clamped)     */

/*
 * Shape and layout of one decode call.
 *
 * K and V caches: element (blk, head, off, i) of K is at
 *   k_cache + blk * k_stride_block + head * k_stride_head + off * k_stride_token + i
 * (same for V with the v_ strides), for blk < num_blocks, head < num_kv_heads,
 * off < block_size, i < head_dim. head_dim is innermost and contiguous. The
 * default layout [num_blocks, num_kv_heads, block_size, head_dim] has strides
 * (H_kv*bs*d, bs*d, d); the token-major layout [num_blocks, block_size,
 * num_kv_heads, head_dim] has (bs*H_kv*d, d, H_kv*d).
 */
typedef struct pa_desc {
  int32_t batch;              /* B, number of sequences (0 is a no-op)            */
  int32_t num_q_heads;        /* H_q                                              */
  int32_t num_kv_heads;       /* H_kv; G = H_q / H_kv                             */
  int32_t head_dim;           /* d: 64, 128 or 256                                */
  int32_t block_size;         /* tokens per physical block, power of two <= 1024  */
  int32_t num_blocks;         /* NB, physical blocks in the pool                  */
  int32_t max_blocks_per_seq; /* MBS, columns of block_table                      */
  int32_t kv_dtype;           /* pa_dtype                                         */
  int64_t k_stride_block, k_stride_head, k_stride_token; /* elements              */
  int64_t v_stride_block, v_stride_head, v_stride_token; /* elements              */
  int32_t partition_size;     /* tokens per KV partition; 0 = library's choice    */
  int32_t path;               /* pa_path                                          */
  int32_t flags;              /* PA_FLAG_* bits                                   */
  int32_t reserved;           /* must be 0                                        */
} pa_desc;

/*
 * Decode attention for one batch, enqueued on `stream` (a hipStream_t; NULL is
 * the default stream). Returns once two kernels are enqueued; it never
 * synchronises the device.
 *
 *   q              float32 [B, H_q, d] (bf16 with PA_FLAG_QO_BF16), contiguous,
 *                  16-byte aligned
 *   k_cache,
 *   v_cache        pools as described at pa_desc, 16-byte aligned
 *   block_table    int32 [B, max_blocks_per_seq], row-major. Only the entries
 *                  j < ceil(L_b / block_size) are read; -1 marks an unassigned
 *                  entry and must not appear in that range.
 *   cache_seqlens  int32 [B], L_b in [0, max_blocks_per_seq * block_size]
 *   scale          multiplies q . k before the softmax (usually 1/sqrt(d))
 *   out            float32 [B, H_q, d] (bf16 with PA_FLAG_QO_BF16), contiguous,
 *                  16-byte aligned; L_b = 0 gives zeros
 *   workspace      device memory of at least paged_attn_workspace_size(desc)
 *                  bytes (may be NULL when that size is 0), 256-byte aligned
 *   status         optional device int32; the kernels OR PA_STATUS_* bits into
 *                  it when a table entry or cache length is invalid. The caller
 *                  clears it. NULL disables the report (invalid entries are still
 *                  never dereferenced).
 *
 * Values inside the device arrays are not checked on the host (that would need a
 * synchronisation); use paged_attn_check_inputs on host copies to vet them.
 * Calls that share a workspace must be ordered on one stream.
 */
int paged_attn_decode(const pa_desc* desc, const void* q, const void* k_cache,
                      const void* v_cache, const int32_t* block_table,
                      const int32_t* cache_seqlens, float scale, void* out, void* workspace,
                      size_t workspace_bytes, int32_t* status, void* stream);

/*
 * paged_attn_decode without a caller workspace, for callers that cannot
 * allocate device memory (code under HIP graph capture, tight serving loops,
 * harnesses that forbid allocation). Same arguments, results and rules as
 * paged_attn_decode, minus workspace and workspace_bytes: the partial states
 * live in a static device array inside the library, PA_STATIC_SCRATCH_BYTES
 * bytes on each device the library runs on, held until the process ends. Its
 * address is looked up once per device, on the first call made with that
 * device current. Nothing is allocated and nothing synchronises; the call
 * enqueues the same kernels as paged_attn_decode on `stream`.
 *
 *   - A descriptor whose paged_attn_workspace_size() exceeds
 *     PA_STATIC_SCRATCH_BYTES returns PA_E_SCRATCH and launches nothing (the
 *     library's own partition choice keeps batches of up to a few million
 *     cached tokens below it; a small explicit partition_size raises the need).
 *   - PA_PATH_MFMA_FUSED returns PA_E_PATH: its arrival counters would have to
 *     be zero in the shared array.
 *   - PA_FLAG_KV_SHARED does not group sequences here (no prefix folding): the
 *     need is the workspace size of the same descriptor without the flag.
 *   - Every call on a device uses that device's one array, which keeps the last
 *     call's contents (no call relies on them). Calls that may overlap in time
 *     on one device -- on different streams, or from several host threads
 *     without ordering -- race on it; order them on one stream.
 *   - PA_E_LAUNCH also reports a failure to look up the array's address.
 */
#define PA_STATIC_SCRATCH_BYTES ((size_t)32 << 20)
int paged_attn_decode_static(const pa_desc* desc, const void* q, const void* k_cache,
                             const void* v_cache, const int32_t* block_table,
                             const int32_t* cache_seqlens, float scale, void* out,
                             int32_t* status, void* stream);

/*
 * The decode step with the new token (page "Paged attention", decoding path:
 * the kernel appends the step's keys and values to the paged cache in place):
 * for every sequence b and KV head, writes k_new[b, h_kv, :] and
 * v_new[b, h_kv, :] at token t = cache_seqlens[b], i.e. block
 * block_table[b][t / block_size], offset t % block_size, then does what
 * paged_attn_decode does over the cache_seqlens[b] + 1 tokens. cache_seqlens is
 * read, not changed (the caller advances it), and block_table must already map
 * the new token's block.
 *
 *   k_new, v_new   [B, H_kv, d], contiguous, the cache's element type, 16-byte
 *                  aligned, device memory owned by the caller
 *   k_cache,
 *   v_cache        written at the new token's slot only
 *   other arguments as for paged_attn_decode
 *
 * Three kernels are enqueued on `stream` (append, partition, combine); nothing
 * is allocated and no memset is issued, so the call can be captured in a HIP
 * graph and replayed with the tensors' contents updated in place between
 * replays. A new token beyond max_blocks_per_seq * block_size, or whose table
 * entry is outside [0, NB), is not written; the status word gets
 * PA_STATUS_BAD_SEQLEN or PA_STATUS_BAD_BLOCK (and the attention clamps or skips
 * that token). Returns the codes of paged_attn_decode, and PA_E_NULL / PA_E_ALIGN
 * for k_new or v_new.
 */
int paged_attn_decode_append(const pa_desc* desc, const void* q, const void* k_new,
                             const void* v_new, void* k_cache, void* v_cache,
                             const int32_t* block_table, const int32_t* cache_seqlens, float scale,
                             void* out, void* workspace, size_t workspace_bytes, int32_t* status,
                             void* stream);

/*
 * The two phases of paged_attn_decode, callable separately (same arguments and
 * rules). paged_attn_partition_phase runs the partition kernel: every
 * (sequence, KV head, partition) folds its tokens into a running softmax state
 * (on the streaming path the split is the waves' equal shares of the batch's
 * 16-token chunks instead: each wave leaves one state per stream it covers
 * only in part); a sequence folded whole by one workgroup or wave gets its
 * normalised output written to out, the others leave their states in the
 * workspace.
 * paged_attn_combine_phase merges those states into out with the max-rescaling
 * combine (page "Paged Attention Kernel Architecture for BI-V100", section 2
 * level 3 and section 6 phase 2) and reads only cache_seqlens and the
 * workspace. Calling the partition phase and then the combine phase on one
 * stream equals paged_attn_decode; the partition phase alone completes out only
 * when paged_attn_workspace_size() is 0, or on PA_PATH_MFMA_FUSED (whose
 * partition kernel merges too). The combine phase is a no-op then.
 */
int paged_attn_partition_phase(const pa_desc* desc, const void* q, const void* k_cache,
                               const void* v_cache, const int32_t* block_table,
                               const int32_t* cache_seqlens, float scale, void* out,
                               void* workspace, size_t workspace_bytes, int32_t* status,
                               void* stream);
int paged_attn_combine_phase(const pa_desc* desc, const int32_t* cache_seqlens, void* out,
                             void* workspace, size_t workspace_bytes, void* stream);

/*
 * Paged varlen prefill (the varlen path of the paged-attention docs page, over
 * the same paged pool as the decode): sequence b owns query rows
 * cu_seqlens_q[b] .. cu_seqlens_q[b+1]-1 of q and attends the seqlens_k[b]
 * tokens its block_table row maps, the new tokens included (written to the
 * cache beforehand). With causal != 0 row i of a sequence with q_len rows and
 * L keys attends tokens [0, L - q_len + i] (bottom-right aligned; a row with
 * none gets zeros), else all L tokens.
 *
 *   desc           batch = number of sequences; heads, head_dim, block_size,
 *                  pool and strides as for the decode. kv_dtype must be f16 or
 *                  bf16 (else PA_E_PATH), block_size >= 16 (else PA_E_SHAPE).
 *                  partition_size and path are ignored; PA_FLAG_QO_BF16 makes q
 *                  and out bf16.
 *   q              float32 [total_q, H_q, d] (total_q = cu_seqlens_q[batch]),
 *                  contiguous, 16-byte aligned
 *   cu_seqlens_q   int32 [batch + 1], cu_seqlens_q[0] = 0, non-decreasing
 *   seqlens_k      int32 [batch], L_b in [0, max_blocks_per_seq * block_size]
 *   max_seqlen_q   an upper bound of every q_len (sizes the grid); a longer
 *                  sequence has its rows past it unwritten and sets
 *                  PA_STATUS_BAD_SEQLEN
 *   out            float32 [total_q, H_q, d], contiguous, 16-byte aligned
 *   workspace      NULL, or device memory of at least
 *                  paged_attn_prefill_workspace_size(desc, max_seqlen_q) bytes
 *                  (smaller: PA_E_WORKSPACE; when that size is not 0, 256-byte
 *                  aligned, else PA_E_ALIGN)
 *                  whose leading paged_attn_prefill_workspace_zeroed_bytes()
 *                  bytes are zero. It holds the key split's arrival counters
 *                  and half states: when the launch's work items (8 (16-row
 *                  tile, head) units each) leave the last round of workgroups
 *                  on the compute units at most half full, that round's items
 *                  run as two halves of their keys, merged by the second half
 *                  to finish (the max-rescaling combine of page "Paged
 *                  Attention Kernel Architecture for BI-V100", section 2).
 *                  Every call leaves the counters zero. NULL (or a size of 0)
 *                  runs every item whole.
 *   workspace_bytes  its size
 *   status         as for the decode (PA_STATUS_BAD_BLOCK, PA_STATUS_BAD_SEQLEN)
 *
 * One launch; asynchronous on `stream`, no allocation (graph-capturable).
 * Calls that share a workspace must be ordered on one stream. Returns PA_OK or
 * a PA_E_* code (nothing launched then).
 */
int paged_attn_prefill(const pa_desc* desc, const void* q, const void* k_cache,
                       const void* v_cache, const int32_t* block_table,
                       const int32_t* cu_seqlens_q, const int32_t* seqlens_k,
                       int32_t max_seqlen_q, int32_t causal, float scale, void* out,
                       void* workspace, size_t workspace_bytes, int32_t* status, void* stream);

/* Bytes of workspace paged_attn_prefill uses for the key split with this
 * descriptor and max_seqlen_q on the current device (the split depends on its
 * compute-unit count); 0 when no work item is split, for a descriptor the
 * prefill refuses and for max_seqlen_q <= 0. */
size_t paged_attn_prefill_workspace_size(const pa_desc* desc, int32_t max_seqlen_q);

/* Leading bytes of that workspace (the arrival counters) that must be zero
 * when a call starts; every call leaves them zero, so zero them once after
 * allocating the workspace or after using it for anything else. */
size_t paged_attn_prefill_workspace_zeroed_bytes(const pa_desc* desc, int32_t max_seqlen_q);

/* Bytes of workspace paged_attn_decode needs for this descriptor on the
 * current device. Grid and VALU kernels: the partial (max, sum, output) of
 * every possible partition, sized from max_blocks_per_seq * block_size; 0 when
 * one partition always suffices. Streaming path (PA_PATH_MFMA_STREAM): two
 * state slots per wave of the kernel's grid, which depends on the device's
 * compute-unit count, and a two-int record per (sequence, KV head); the
 * partition size does not enter. With PA_FLAG_KV_SHARED grouping (see the
 * flag) also a record per (group, KV head), the slots' rows sized for the F x G
 * columns, the groups' lengths and one state's rows per stream. MFMA_FUSED: its arrival counters first (see
 * pa_path). Otherwise the contents need no initialisation and carry nothing
 * between calls. Returns 0 for an invalid descriptor too; call
 * paged_attn_validate first. */
size_t paged_attn_workspace_size(const pa_desc* desc);

/* Checks the descriptor alone (host only, no device access). PA_OK or PA_E_*. */
int paged_attn_validate(const pa_desc* desc);

/* The partition size paged_attn_decode will use (tokens), or a negative PA_E_*.
 * The streaming path splits by the waves' shares and does not use it. */
int paged_attn_partition_size(const pa_desc* desc);

/* The kernel paged_attn_decode will run (PA_PATH_VALU, PA_PATH_MFMA_GRID or
 * PA_PATH_MFMA_STREAM), or a negative PA_E_* when the descriptor is invalid. */
int paged_attn_resolved_path(const pa_desc* desc);

/* Host-side, synchronous check of the device arrays' VALUES on host copies:
 * every cache length in [0, MBS * bs] and every table entry read for an
 * attended token in [0, num_blocks). Returns PA_OK, PA_E_SEQLEN or PA_E_TABLE
 * (or a descriptor error). Touches no device. */
int paged_attn_check_inputs(const pa_desc* desc, const int32_t* block_table_host,
                            const int32_t* cache_seqlens_host);

/* Static text for a status code. */
const char* paged_attn_strerror(int status);

/* PA_ABI_VERSION of the built library. */
int paged_attn_abi_version(void);

#ifdef __cplusplus
}
#endif

#endif /* PAGED_ATTN_H */
