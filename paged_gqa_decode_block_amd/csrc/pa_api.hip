// pa_api.hip -- the extern "C" entry points declared in include/paged_attn.h:
// descriptor validation, workspace sizing, path and partition-size selection,
// host-side value checks, and the two launches of a decode call.
#include <stdlib.h>
#include <string.h>

#include <mutex>

#include "../../include/paged_attn.h"
#include "pa_kernels.h"

namespace {

bool is_pow2(int x) { return x > 0 && (x & (x - 1)) == 0; }

int ilog2(int x) {
  int r = 0;
  while ((1 << r) < x) ++r;
  return r;
}

int elem_bytes(int dtype) { return dtype == PA_DTYPE_F32 ? 4 : 2; }

size_t align256(size_t x) { return (x + 255) & ~(size_t)255; }

int64_t max_tokens(const pa_desc* d) { return (int64_t)d->max_blocks_per_seq * d->block_size; }

int pick_path(const pa_desc* d);
bool stream_pays(const pa_desc* d);
int cu_count();
int stream_variant();
int stream_variant_for(const pa_desc* d);

// Partition size for a descriptor that passed validation of everything else.
// Without a caller choice: 4096 tokens for the streaming kernel (its waves
// split the work by chunks, so the partition size only sets how many partial
// states are written and merged); for the merged grid variant the rule below;
// for the other kernels 512, halved (down to 64) while the busiest possible
// grid would hold fewer than 1024 work items.
int pick_partition(const pa_desc* d) {
  if (d->partition_size > 0) return d->partition_size;
  const int64_t T = max_tokens(d);
  if (pick_path(d) == PA_PATH_MFMA_STREAM) {
    int part = 4096;
    while ((part >> ilog2(d->block_size)) + 2 > pa::kTableCap && part > 32) part >>= 1;
    return part;
  }
  if (pick_path(d) == PA_PATH_MFMA_FUSED) {
    // Fewer, longer partitions: the merge reads every partition state of a KV
    // head in one wave. 1024, halved while the busiest grid would hold fewer
    // than 1024 work items but not below min(1024, max_tokens / 16), then
    // doubled while the merge state would not fit in LDS.
    const int64_t lo = T / 16 < 1024 ? T / 16 : 1024;
    const int G = d->num_q_heads / d->num_kv_heads;
    int part = 1024;
    while (part > 64 && part / 2 >= lo &&
           (int64_t)d->batch * d->num_kv_heads * ((T + part - 1) / part) < 1024)
      part >>= 1;
    while (part < 16384 &&
           2 * ((T + part - 1) / part) * G + 16 > pa::fused_merge_capacity(d->head_dim))
      part <<= 1;
    while ((part >> ilog2(d->block_size)) + 2 > pa::kTableCap && part > 32) part >>= 1;
    return part;
  }
  int part = 512;
  while (part > 64 && (int64_t)d->batch * d->num_kv_heads * ((T + part - 1) / part) < 1024)
    part >>= 1;
  // keep within the LDS block-id table
  while ((part >> ilog2(d->block_size)) + 2 > pa::kTableCap && part > 32) part >>= 1;
  return part;
}

// Whether the persistent streaming kernel beats the one-workgroup-per-
// partition grid kernel: only on batches whose K/V (bounded by
// max_blocks_per_seq * block_size tokens per sequence) reaches 160 MB. Below
// that each persistent wave gets a short share and its start-up (lengths,
// table, then K/V, about 10 us) is not amortised, while the grid kernel starts
// every partition at once. On one MI355X the grid kernel took 0.6-0.9x the
// streaming kernel's time up to 128 MB; from 192 MB the streaming kernel was
// faster in three of four shapes and from 320 MB in all.
bool stream_pays(const pa_desc* d) {
  const int64_t elem = d->kv_dtype == PA_DTYPE_F32 ? 4 : 2;
  const int64_t bytes = (int64_t)d->batch * d->num_kv_heads * max_tokens(d) * d->head_dim * elem * 2;
  return bytes >= ((int64_t)160 << 20);
}

// The kernel a descriptor runs on: PA_PATH_VALU, PA_PATH_MFMA_GRID or
// PA_PATH_MFMA_STREAM (or an error).
int pick_path(const pa_desc* d) {
  const int G = d->num_q_heads / d->num_kv_heads;
  // the x-packed K / transposed V layout is read by the grid kernel only
  const bool xp = (d->flags & PA_FLAG_KV_XPACKED) != 0;
  // the streaming kernel counts a batch's 16-token chunks (all KV heads) in 32 bits
  const bool stream_ok =
      !xp && pa::stream_supports(d->kv_dtype, d->head_dim, G, d->block_size, d->batch) &&
      (int64_t)d->batch * d->num_kv_heads * ((max_tokens(d) + 15) / 16) < ((int64_t)1 << 31);
  switch (d->path) {
    case PA_PATH_VALU:
      if (xp) return PA_E_PATH;
      return pa::valu_supports(d->kv_dtype, d->head_dim, G) ? PA_PATH_VALU : PA_E_SHAPE;
    case PA_PATH_MFMA:
    case PA_PATH_MFMA_GRID:
    case PA_PATH_MFMA_STREAM:
    case PA_PATH_MFMA_FUSED:
      if (d->kv_dtype == PA_DTYPE_F32) return PA_E_PATH;
      if (!pa::mfma_supports(d->kv_dtype, d->head_dim, G)) return PA_E_SHAPE;
      if (d->path == PA_PATH_MFMA_GRID || d->path == PA_PATH_MFMA_FUSED) return d->path;
      if (d->path == PA_PATH_MFMA_STREAM) return stream_ok ? PA_PATH_MFMA_STREAM : PA_E_PATH;
      return stream_ok && stream_pays(d) ? PA_PATH_MFMA_STREAM : PA_PATH_MFMA_GRID;
  }
  // AUTO: matrix cores for 16-bit K/V, vector ALUs for fp32
  if (d->kv_dtype != PA_DTYPE_F32 && pa::mfma_supports(d->kv_dtype, d->head_dim, G))
    return stream_ok && stream_pays(d) ? PA_PATH_MFMA_STREAM : PA_PATH_MFMA_GRID;
  if (xp) return PA_E_PATH;
  if (pa::valu_supports(d->kv_dtype, d->head_dim, G)) return PA_PATH_VALU;
  return PA_E_SHAPE;
}

// Ring depth / occupancy variant of the streaming kernel: PAGEDATTN_STREAM_VARIANT
// (0 to 3; read once) for tuning sweeps, 0 otherwise.
int stream_variant() {
  static int v = -1;
  if (v < 0) {
    const char* e = getenv("PAGEDATTN_STREAM_VARIANT");
    v = (e && e[0] >= '0' && e[0] <= '3') ? e[0] - '0' : 0;
  }
  return v;
}

// The variant a call runs: bf16 q/out is built for the default variant only.
int stream_variant_for(const pa_desc* d) { return (d->flags & PA_FLAG_QO_BF16) ? 0 : stream_variant(); }

// Non-temporal K/V loads in the streaming kernel (unless the descriptor says
// blocks are shared): PAGEDATTN_STREAM_NT=0 turns them off for tuning sweeps
// (read once), on otherwise.
bool stream_nt() {
  static int v = -1;
  if (v < 0) {
    const char* e = getenv("PAGEDATTN_STREAM_NT");
    v = (e && e[0] == '0') ? 0 : 1;
  }
  return v == 1;
}

// Grid of the streaming kernel for a descriptor on the current device: it
// bounds the chunks of work by max_blocks_per_seq * block_size tokens per
// sequence.
int stream_waves(const pa_desc* d) {
  const int64_t chunks_per_stream = (max_tokens(d) + 15) / 16;
  return pa::stream_grid(d->head_dim, stream_variant_for(d), cu_count(),
                         (int64_t)d->batch * d->num_kv_heads * chunks_per_stream);
}

// Compute units of the current device (cached per device).
int cu_count() {
  static int cache[64] = {0};
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return 256;
  if (cache[dev] == 0) {
    int n = 0;
    if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || n <= 0)
      n = 256;
    cache[dev] = n;
  }
  return cache[dev];
}

int validate(const pa_desc* d) {
  if (!d) return PA_E_NULL;
  if (d->batch < 0 || d->num_q_heads <= 0 || d->num_kv_heads <= 0 || d->num_blocks <= 0 ||
      d->max_blocks_per_seq <= 0)
    return PA_E_SHAPE;
  if (d->num_q_heads % d->num_kv_heads) return PA_E_SHAPE;
  // grid dimensions y and z carry heads and sequences
  if (d->batch > 65535 || d->num_q_heads > 65535) return PA_E_SHAPE;
  if (d->head_dim != 64 && d->head_dim != 128 && d->head_dim != 256) return PA_E_HEAD_DIM;
  if (!is_pow2(d->block_size) || d->block_size > 1024) return PA_E_BLOCK_SIZE;
  if (d->kv_dtype != PA_DTYPE_F32 && d->kv_dtype != PA_DTYPE_F16 && d->kv_dtype != PA_DTYPE_BF16)
    return PA_E_DTYPE;
  if (max_tokens(d) > (int64_t)1 << 30) return PA_E_SHAPE;
  const int64_t eb = elem_bytes(d->kv_dtype);
  const bool xp = (d->flags & PA_FLAG_KV_XPACKED) != 0;
  const int64_t st[6] = {d->k_stride_block, d->k_stride_head, d->k_stride_token,
                         d->v_stride_block, d->v_stride_head, d->v_stride_token};
  for (int i = 0; i < 6; ++i)
    if (st[i] <= 0 || (!(xp && i % 3 == 2) && (st[i] * eb) % 16)) return PA_E_STRIDE;
  if (xp) {
    // dense [d/x, bs, x] and [d, bs] tiles of 16-bit elements (x = 8); a piece
    // of V^T is 8 consecutive tokens of one block, hence block_size >= 8
    if (d->kv_dtype == PA_DTYPE_F32) return PA_E_PATH;
    if (d->block_size < 8) return PA_E_BLOCK_SIZE;
    if (d->k_stride_token != 8 || d->v_stride_token != 1) return PA_E_STRIDE;
    const int64_t tile = (int64_t)d->block_size * d->head_dim;
    if (d->k_stride_head < tile || d->v_stride_head < tile) return PA_E_STRIDE;
  } else if (d->k_stride_token < d->head_dim || d->v_stride_token < d->head_dim) {
    return PA_E_STRIDE;
  }
  if (d->path < PA_PATH_AUTO || d->path > PA_PATH_MFMA_FUSED) return PA_E_PATH;
  if ((d->flags & ~(PA_FLAG_KV_SHARED | PA_FLAG_QO_BF16 | PA_FLAG_KV_XPACKED)) || d->reserved)
    return PA_E_SHAPE;
  if (d->partition_size != 0) {
    const int ps = d->partition_size;
    if (ps < 32 || ps > 16384 || ps % 32) return PA_E_PARTITION;
    if ((ps >> ilog2(d->block_size)) + 2 > pa::kTableCap) return PA_E_PARTITION;
  }
  // the partition index is grid dimension y
  if ((max_tokens(d) + pick_partition(d) - 1) / pick_partition(d) > 65535) return PA_E_PARTITION;
  const int path = pick_path(d);
  if (path < 0) return path;
  // the merged variant keeps every partition's max, sum and weight in LDS
  if (path == PA_PATH_MFMA_FUSED) {
    const int part = pick_partition(d);
    const int64_t pmax = (max_tokens(d) + part - 1) / part;
    if (2 * pmax * (d->num_q_heads / d->num_kv_heads) + 16 > pa::fused_merge_capacity(d->head_dim))
      return PA_E_PARTITION;
  }
  return PA_OK;
}

// Prefix folding (streaming path, blocks shared between sequences): groups of
// F = 16 / G consecutive sequences (G <= 8), whose shared leading blocks are
// read once with the F x G query heads in the score MFMA's 16 columns. 0 when
// it does not apply: another path, no sharing declared, G > 8, or more
// virtual sequences (groups x (F + 1)) than the kernel's 1024. The
// PAGEDATTN_FOLD=0 environment switch (read once) turns it off for A/B runs.
int fold_enabled() {
  static int v = -1;
  if (v < 0) {
    const char* e = getenv("PAGEDATTN_FOLD");
    v = (e && e[0] == '0') ? 0 : 1;
  }
  return v;
}
int fold_factor(const pa_desc* d) {
  if (!(d->flags & PA_FLAG_KV_SHARED) || !fold_enabled() || d->batch < 2) return 0;
  if (pick_path(d) != PA_PATH_MFMA_STREAM) return 0;
  const int G = d->num_q_heads / d->num_kv_heads;
  const int F = 16 / G;
  if (F < 2) return 0;
  const int64_t groups = ((int64_t)d->batch + F - 1) / F;
  if (groups * (F + 1) > 1024) return 0;
  return F;
}

// Workspace regions of a valid descriptor, as byte offsets (each 256-byte
// aligned; off[kWsParts] is the total): for the merged grid variant first an
// arrival word per (sequence, KV head) (at offset 0 for every descriptor; zero
// before the first call and left zero by every call); for the grid and VALU
// kernels the partition states m, l, acc of every (sequence, query head,
// partition), nothing when one partition always suffices; for the streaming
// kernel a record per (sequence, KV head) stream and two state slots (m, l and
// acc of the G heads, or with folding of the F x G prefix columns) per wave of
// its grid (per pair of waves at head_dim 256), and with folding a record per
// (group, KV head) prefix stream, the F + 1 virtual sequences' lengths of
// each group (its prefix, then each member past it) and state rows of every
// stream for the ones that lie inside one share but are not written out.
enum { kWsCnt, kWsM, kWsL, kWsAcc, kWsLink, kWsCm, kWsCl, kWsCacc, kWsPre, kWsOm, kWsOl, kWsOacc,
       kWsParts };
void workspace_layout(const pa_desc* d, size_t* off, int fold) {
  const int part = pick_partition(d);
  const int64_t pmax = (max_tokens(d) + part - 1) / part;
  const bool stream = pick_path(d) == PA_PATH_MFMA_STREAM;
  size_t sz[kWsParts] = {0};
  if (stream) {
    const int G = d->num_q_heads / d->num_kv_heads;
    const size_t rps = fold > 0 ? (size_t)fold * G : (size_t)G;
    const size_t groups = fold > 0 ? ((size_t)d->batch + fold - 1) / fold : 0;
    const size_t slots = 2 * (size_t)stream_waves(d);
    sz[kWsLink] = ((size_t)d->batch + groups) * d->num_kv_heads * 2 * sizeof(int32_t);
    sz[kWsCm] = sz[kWsCl] = slots * rps * sizeof(float);
    sz[kWsCacc] = slots * rps * d->head_dim * sizeof(float);
    sz[kWsPre] = groups * (fold + 1) * sizeof(int32_t);
    if (fold > 0) {
      const size_t orows = ((size_t)d->batch + groups) * d->num_kv_heads * rps;
      sz[kWsOm] = sz[kWsOl] = orows * sizeof(float);
      sz[kWsOacc] = orows * d->head_dim * sizeof(float);
    }
  } else if (pmax > 1) {
    const size_t rows = (size_t)d->batch * d->num_q_heads * (size_t)pmax;
    sz[kWsM] = sz[kWsL] = rows * sizeof(float);
    sz[kWsAcc] = rows * d->head_dim * sizeof(float);
  }
  if (pick_path(d) == PA_PATH_MFMA_FUSED && pmax > 1)
    sz[kWsCnt] = (size_t)d->batch * d->num_kv_heads * sizeof(int32_t);
  off[0] = 0;
  for (int i = 0; i < kWsParts; ++i) off[i + 1] = off[i] + align256(sz[i]);
}

// Stripe-count hint for the combine after the streaming kernel: about how many
// waves' states a stream has when every sequence is as long as the table
// allows (longest stream over the average share), doubled with room for
// shorter shares. It only sizes the combine's workgroups; any count is merged.
int stream_states_hint(const pa_desc* d, int waves) {
  const int64_t per_stream = (max_tokens(d) + 15) / 16;
  const int64_t total = (int64_t)d->batch * d->num_kv_heads * per_stream;
  const int64_t share = total / (waves > 0 ? waves : 1);
  const int64_t n = per_stream / (share > 0 ? share : 1) + 1;
  const int64_t hint = 2 * n + 2;
  return (int)(hint < waves ? hint : waves);
}

}  // namespace

extern "C" {

int paged_attn_abi_version(void) { return PA_ABI_VERSION; }

int paged_attn_validate(const pa_desc* desc) { return validate(desc); }

int paged_attn_partition_size(const pa_desc* desc) {
  const int rc = validate(desc);
  return rc != PA_OK ? rc : pick_partition(desc);
}

int paged_attn_resolved_path(const pa_desc* desc) {
  const int rc = validate(desc);
  return rc != PA_OK ? rc : pick_path(desc);
}

size_t paged_attn_workspace_size(const pa_desc* desc) {
  if (validate(desc) != PA_OK) return 0;
  size_t off[kWsParts + 1];
  workspace_layout(desc, off, fold_factor(desc));
  return off[kWsParts];
}

namespace {
// the prefill launch's parameters that size its workspace
pa::Params prefill_shape(const pa_desc* desc) {
  pa::Params p{};
  p.B = desc->batch;
  p.Hq = desc->num_q_heads;
  p.Hkv = desc->num_kv_heads;
  p.G = desc->num_q_heads / desc->num_kv_heads;
  p.D = desc->head_dim;
  p.qo_bf16 = (desc->flags & PA_FLAG_QO_BF16) ? 1 : 0;
  p.cus = cu_count();
  return p;
}
bool prefill_kv_ok(const pa_desc* desc) {
  return desc->kv_dtype != PA_DTYPE_F32 && !(desc->flags & PA_FLAG_KV_XPACKED) &&
         desc->block_size >= 16;
}
}  // namespace

size_t paged_attn_prefill_workspace_size(const pa_desc* desc, int32_t max_seqlen_q) {
  if (validate(desc) != PA_OK || !prefill_kv_ok(desc) || max_seqlen_q <= 0) return 0;
  return pa::prefill_workspace_bytes(prefill_shape(desc), desc->kv_dtype, max_seqlen_q);
}

size_t paged_attn_prefill_workspace_zeroed_bytes(const pa_desc* desc, int32_t max_seqlen_q) {
  if (validate(desc) != PA_OK || !prefill_kv_ok(desc) || max_seqlen_q <= 0) return 0;
  return pa::prefill_workspace_zeroed_bytes(prefill_shape(desc), desc->kv_dtype, max_seqlen_q);
}

int paged_attn_check_inputs(const pa_desc* desc, const int32_t* table, const int32_t* seqlens) {
  const int rc = validate(desc);
  if (rc != PA_OK) return rc;
  if (desc->batch > 0 && (!table || !seqlens)) return PA_E_NULL;
  const int64_t lmax = max_tokens(desc);
  for (int b = 0; b < desc->batch; ++b) {
    const int L = seqlens[b];
    if (L < 0 || L > lmax) return PA_E_SEQLEN;
    const int nblk = (L + desc->block_size - 1) / desc->block_size;
    const int32_t* row = table + (int64_t)b * desc->max_blocks_per_seq;
    for (int j = 0; j < nblk; ++j)
      if (row[j] < 0 || row[j] >= desc->num_blocks) return PA_E_TABLE;
  }
  return PA_OK;
}

const char* paged_attn_strerror(int status) {
  switch (status) {
    case PA_OK: return "ok";
    case PA_E_NULL: return "a required pointer is NULL";
    case PA_E_SHAPE: return "unsupported or inconsistent sizes (batch, heads, blocks, or G for this path)";
    case PA_E_HEAD_DIM: return "head_dim must be 64, 128 or 256";
    case PA_E_BLOCK_SIZE: return "block_size must be a power of two in [1, 1024]";
    case PA_E_DTYPE: return "kv_dtype must be PA_DTYPE_F32, PA_DTYPE_F16 or PA_DTYPE_BF16";
    case PA_E_STRIDE: return "K/V strides must be positive multiples of 16 bytes, token stride >= head_dim";
    case PA_E_ALIGN: return "q, out, k_cache and v_cache must be 16-byte aligned";
    case PA_E_PARTITION: return "partition_size must be 0 or a multiple of 32 in [32, 16384] spanning <= 1022 blocks (MFMA_FUSED: 2 * n_part * G + 16 <= 16 * head_dim)";
    case PA_E_WORKSPACE: return "workspace missing or smaller than paged_attn_workspace_size()";
    case PA_E_PATH: return "path must be a pa_path; the MFMA path needs f16 or bf16 K/V; the x-packed K/V layout runs on MFMA_GRID or MFMA_FUSED only";
    case PA_E_LAUNCH: return "the HIP runtime refused a kernel launch";
    case PA_E_TABLE: return "a block_table entry for an attended token is outside [0, num_blocks)";
    case PA_E_SEQLEN: return "a cache length is negative or beyond max_blocks_per_seq * block_size";
    case PA_E_NOMEM: return "not enough free blocks in the block manager";
    case PA_E_SEQ: return "unknown sequence, or a block index or length outside it";
    case PA_E_SCRATCH: return "the call needs more workspace than the library's static scratch (PA_STATIC_SCRATCH_BYTES) holds; pass a workspace to paged_attn_decode instead";
  }
  return "unknown status";
}

}  // extern "C"

namespace {

// Shared argument checks and parameter set-up of the decode entry points.
// Returns PA_OK and fills p, or an error code.
int prepare(const pa_desc* desc, const void* q, const void* k_cache, const void* v_cache,
            const int32_t* block_table, const int32_t* cache_seqlens, float scale, void* out,
            void* workspace, size_t workspace_bytes, int32_t* status, bool need_inputs,
            pa::Params& p, bool need_ws = true, bool allow_fold = true) {
  int rc = validate(desc);
  if (rc != PA_OK) return rc;
  memset(&p, 0, sizeof p);
  p.B = desc->batch;
  if (desc->batch == 0) return PA_OK;
  if (!cache_seqlens || !out) return PA_E_NULL;
  if (need_inputs && (!q || !k_cache || !v_cache || !block_table)) return PA_E_NULL;
  if (((uintptr_t)q | (uintptr_t)k_cache | (uintptr_t)v_cache | (uintptr_t)out) & 15) return PA_E_ALIGN;
  const int fold = allow_fold ? fold_factor(desc) : 0;
  size_t off[kWsParts + 1];
  workspace_layout(desc, off, fold);
  const size_t need = need_ws ? off[kWsParts] : 0;
  if (need > 0 && (!workspace || workspace_bytes < need || ((uintptr_t)workspace & 255)))
    return PA_E_WORKSPACE;

  const int part = pick_partition(desc);
  p.q = q;
  p.k = k_cache;
  p.v = v_cache;
  p.table = block_table;
  p.seqlens = cache_seqlens;
  p.out = out;
  p.status = status;
  p.ksb = desc->k_stride_block;
  p.ksh = desc->k_stride_head;
  p.kst = desc->k_stride_token;
  p.vsb = desc->v_stride_block;
  p.vsh = desc->v_stride_head;
  p.vst = desc->v_stride_token;
  p.Hq = desc->num_q_heads;
  p.Hkv = desc->num_kv_heads;
  p.G = desc->num_q_heads / desc->num_kv_heads;
  p.D = desc->head_dim;
  p.bs_log2 = ilog2(desc->block_size);
  p.NB = desc->num_blocks;
  p.MBS = desc->max_blocks_per_seq;
  p.part = part;
  p.pmax = (int)((max_tokens(desc) + part - 1) / part);
  p.qscale = scale * 1.4426950408889634f;  // log2(e): scores in base-2 units
  p.cus = cu_count();
  p.qo_bf16 = (desc->flags & PA_FLAG_QO_BF16) ? 1 : 0;
  p.xpacked = (desc->flags & PA_FLAG_KV_XPACKED) ? 1 : 0;
  p.rps = p.G;
  if (need > 0) {
    char* ws = (char*)workspace;
    if (pick_path(desc) == PA_PATH_MFMA_STREAM) {
      if (fold > 0) {
        p.fold = fold;
        p.rps = fold * p.G;
        p.ws_vlen = (int32_t*)(ws + off[kWsPre]);
        p.ws_om = (float*)(ws + off[kWsOm]);
        p.ws_ol = (float*)(ws + off[kWsOl]);
        p.ws_oacc = (float*)(ws + off[kWsOacc]);
      }
      p.ws_link = (int32_t*)(ws + off[kWsLink]);
      p.ws_cm = (float*)(ws + off[kWsCm]);
      p.ws_cl = (float*)(ws + off[kWsCl]);
      p.ws_cacc = (float*)(ws + off[kWsCacc]);
      p.nwaves = stream_waves(desc);
      p.pmax = stream_states_hint(desc, p.nwaves);
    } else {
      p.ws_m = (float*)(ws + off[kWsM]);
      p.ws_l = (float*)(ws + off[kWsL]);
      p.ws_acc = (float*)(ws + off[kWsAcc]);
    }
    if (pick_path(desc) == PA_PATH_MFMA_FUSED && p.pmax > 1) p.ws_cnt = (int32_t*)(ws + off[kWsCnt]);
  }
  return PA_OK;
}

int run_partition(const pa_desc* desc, const pa::Params& p, hipStream_t s) {
  hipError_t e;
  switch (pick_path(desc)) {
    case PA_PATH_MFMA_STREAM:
      e = pa::launch_fold_scan(p, s);
      if (e == hipSuccess)
        e = pa::launch_partition_stream(p, desc->kv_dtype, stream_variant_for(desc),
                                        !(desc->flags & PA_FLAG_KV_SHARED) && stream_nt(), s);
      break;
    case PA_PATH_MFMA_GRID:
    case PA_PATH_MFMA_FUSED: e = pa::launch_partition_mfma(p, desc->kv_dtype, s); break;
    default: e = pa::launch_partition_valu(p, desc->kv_dtype, s); break;
  }
  return e == hipSuccess ? PA_OK : PA_E_LAUNCH;
}

int run_combine(const pa::Params& p, hipStream_t s) {
  // without links (kernels other than the streaming one) a single partition
  // was written out already; the merged grid variant has no second kernel
  if ((p.pmax <= 1 && !p.ws_link) || p.ws_cnt) return PA_OK;
  return pa::launch_combine(p, s) == hipSuccess ? PA_OK : PA_E_LAUNCH;
}

int decode_impl(const pa_desc* desc, const void* q, const void* k_cache, const void* v_cache,
                const int32_t* block_table, const int32_t* cache_seqlens, float scale, void* out,
                void* workspace, size_t workspace_bytes, int32_t* status, void* stream,
                bool allow_fold) {
  pa::Params p;
  int rc = prepare(desc, q, k_cache, v_cache, block_table, cache_seqlens, scale, out, workspace,
                   workspace_bytes, status, true, p, true, allow_fold);
  if (rc != PA_OK || p.B == 0) return rc;
  rc = run_partition(desc, p, (hipStream_t)stream);
  if (rc != PA_OK) return rc;
  return run_combine(p, (hipStream_t)stream);
}

}  // namespace

extern "C" {

int paged_attn_decode(const pa_desc* desc, const void* q, const void* k_cache, const void* v_cache,
                      const int32_t* block_table, const int32_t* cache_seqlens, float scale,
                      void* out, void* workspace, size_t workspace_bytes, int32_t* status,
                      void* stream) {
  return decode_impl(desc, q, k_cache, v_cache, block_table, cache_seqlens, scale, out, workspace,
                     workspace_bytes, status, stream, true);
}

}  // extern "C"

// ---- the allocation-free decode ---------------------------------------------
// The library's own workspace for paged_attn_decode_static: one static array per
// device, zero-initialised when the code object is loaded, held until the
// process ends. Host code never passes the array's name to a kernel (on the host
// it is a stand-in, not a device address); it uses the address that
// hipGetSymbolAddress returns for the current device, looked up once per device.
namespace {

static __device__ __align__(256) unsigned char scratch[PA_STATIC_SCRATCH_BYTES];

constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void* g_scratch_ptr[kMaxDevices];

// Address of the current device's scratch array, or nullptr when the runtime
// cannot say which device is current or where the array is.
void* scratch_for_current_device() {
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return nullptr;
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (!g_scratch_ptr[dev]) {
    void* ptr = nullptr;
    if (hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch)) != hipSuccess || !ptr) return nullptr;
    g_scratch_ptr[dev] = ptr;
  }
  return g_scratch_ptr[dev];
}

}  // namespace

extern "C" {

int paged_attn_decode_static(const pa_desc* desc, const void* q, const void* k_cache,
                             const void* v_cache, const int32_t* block_table,
                             const int32_t* cache_seqlens, float scale, void* out,
                             int32_t* status, void* stream) {
  const int rc = validate(desc);
  if (rc != PA_OK) return rc;
  // the merged grid variant keeps arrival counters that would have to be zero
  if (pick_path(desc) == PA_PATH_MFMA_FUSED) return PA_E_PATH;
  // without prefix folding: its state rows would not fit the scratch for
  // batches that the unfolded layout does
  size_t off[kWsParts + 1];
  workspace_layout(desc, off, 0);
  const size_t need = off[kWsParts];
  if (need > PA_STATIC_SCRATCH_BYTES) return PA_E_SCRATCH;
  void* ws = nullptr;
  if (need > 0 && desc->batch > 0) {
    ws = scratch_for_current_device();
    if (!ws) return PA_E_LAUNCH;
  }
  return decode_impl(desc, q, k_cache, v_cache, block_table, cache_seqlens, scale, out, ws,
                     need > 0 ? PA_STATIC_SCRATCH_BYTES : 0, status, stream, false);
}

int paged_attn_decode_append(const pa_desc* desc, const void* q, const void* k_new,
                             const void* v_new, void* k_cache, void* v_cache,
                             const int32_t* block_table, const int32_t* cache_seqlens, float scale,
                             void* out, void* workspace, size_t workspace_bytes, int32_t* status,
                             void* stream) {
  pa::Params p;
  int rc = prepare(desc, q, k_cache, v_cache, block_table, cache_seqlens, scale, out, workspace,
                   workspace_bytes, status, true, p);
  if (rc != PA_OK || p.B == 0) return rc;
  if (!k_new || !v_new) return PA_E_NULL;
  if (((uintptr_t)k_new | (uintptr_t)v_new) & 15) return PA_E_ALIGN;
  p.len_add = 1;  // the new token is attended too
  const hipStream_t s = (hipStream_t)stream;
  if (pa::launch_append(p, k_new, v_new, elem_bytes(desc->kv_dtype), s) != hipSuccess)
    return PA_E_LAUNCH;
  rc = run_partition(desc, p, s);
  if (rc != PA_OK) return rc;
  return run_combine(p, s);
}

int paged_attn_partition_phase(const pa_desc* desc, const void* q, const void* k_cache,
                               const void* v_cache, const int32_t* block_table,
                               const int32_t* cache_seqlens, float scale, void* out,
                               void* workspace, size_t workspace_bytes, int32_t* status,
                               void* stream) {
  pa::Params p;
  const int rc = prepare(desc, q, k_cache, v_cache, block_table, cache_seqlens, scale, out,
                         workspace, workspace_bytes, status, true, p);
  if (rc != PA_OK || p.B == 0) return rc;
  return run_partition(desc, p, (hipStream_t)stream);
}

int paged_attn_prefill(const pa_desc* desc, const void* q, const void* k_cache, const void* v_cache,
                       const int32_t* block_table, const int32_t* cu_seqlens_q,
                       const int32_t* seqlens_k, int32_t max_seqlen_q, int32_t causal, float scale,
                       void* out, void* workspace, size_t workspace_bytes, int32_t* status,
                       void* stream) {
  pa::Params p;
  const int rc = prepare(desc, q, k_cache, v_cache, block_table, seqlens_k, scale, out, nullptr, 0,
                         status, true, p, false);
  if (rc != PA_OK || p.B == 0) return rc;
  if (!cu_seqlens_q) return PA_E_NULL;
  if (desc->kv_dtype == PA_DTYPE_F32 || (desc->flags & PA_FLAG_KV_XPACKED)) return PA_E_PATH;
  if (desc->block_size < 16 || max_seqlen_q < 0) return PA_E_SHAPE;
  if (max_seqlen_q == 0) return PA_OK;
  // the key split needs its workspace; without one every work item runs whole
  const size_t need = pa::prefill_workspace_bytes(p, desc->kv_dtype, max_seqlen_q);
  if (workspace && need > workspace_bytes) return PA_E_WORKSPACE;
  if (workspace && need > 0 && ((uintptr_t)workspace & 255)) return PA_E_ALIGN;
  return pa::launch_prefill(p, desc->kv_dtype, cu_seqlens_q, max_seqlen_q, causal != 0,
                            need > 0 ? workspace : nullptr, (hipStream_t)stream) == hipSuccess
             ? PA_OK
             : PA_E_LAUNCH;
}

int paged_attn_combine_phase(const pa_desc* desc, const int32_t* cache_seqlens, void* out,
                             void* workspace, size_t workspace_bytes, void* stream) {
  pa::Params p;
  const int rc = prepare(desc, nullptr, nullptr, nullptr, nullptr, cache_seqlens, 1.f, out,
                         workspace, workspace_bytes, nullptr, false, p);
  if (rc != PA_OK || p.B == 0) return rc;
  return run_combine(p, (hipStream_t)stream);
}

}  // extern "C"
