// pa_block_manager.hip -- host-side physical block manager (free list,
// reference counts, per-sequence block lists, prefix sharing, copy-on-write)
// and the device copy of copy-on-write blocks. The operations follow page
// "paged-attention-runtime" (design notes, BlockManager); the interface is
// include/paged_block_manager.h.
#include <new>
#include <unordered_map>
#include <vector>

#include "paged_block_manager.h"
#include "pa_kernels.h"

struct pa_block_manager {
  int32_t num_blocks = 0;
  int32_t block_size = 0;
  std::vector<int32_t> free_list;  // a stack: back() is the next block handed out
  std::vector<int32_t> ref;        // reference count per block
  std::unordered_map<int64_t, std::vector<int32_t>> seqs;

  int32_t take() {  // a free block with one reference (caller checked free_list)
    const int32_t b = free_list.back();
    free_list.pop_back();
    ref[b] = 1;
    return b;
  }
  void drop(int32_t b) {  // one reference less; back to the free list at zero
    if (--ref[b] == 0) free_list.push_back(b);
  }
};

namespace {

bool pow2(int32_t x) { return x > 0 && (x & (x - 1)) == 0; }

// The device copy of copy-on-write: workgroup (pair, KV head) copies that head's
// block_size rows of d elements from block src to block dst, 16 bytes a thread
// (with the x-packed layout a (block, head) tile is block_size * d dense
// elements, copied as rows of d).
__global__ void __launch_bounds__(256)
copy_blocks_kernel(pa::Params p, const int32_t* pairs, int elem_bytes) {
  const int src = pairs[2 * blockIdx.x], dst = pairs[2 * blockIdx.x + 1];
  if (src < 0 || src >= p.NB || dst < 0 || dst >= p.NB) {
    if (threadIdx.x == 0 && blockIdx.y == 0 && p.status) atomicOr(p.status, pa::kStatusBadBlock);
    return;
  }
  const int hk = blockIdx.y;
  const int bs = 1 << p.bs_log2;
  const int vec = p.D * elem_bytes / 16;  // 16-byte pieces per row
  char* k = (char*)p.k;
  char* v = (char*)p.v;
  for (int i = threadIdx.x; i < bs * vec; i += blockDim.x) {
    const int t = i / vec, c = i - t * vec;
    const int64_t ks = ((int64_t)src * p.ksb + hk * p.ksh + t * p.kst) * elem_bytes + 16 * c;
    const int64_t kd = ((int64_t)dst * p.ksb + hk * p.ksh + t * p.kst) * elem_bytes + 16 * c;
    const int64_t vs = ((int64_t)src * p.vsb + hk * p.vsh + t * p.vst) * elem_bytes + 16 * c;
    const int64_t vd = ((int64_t)dst * p.vsb + hk * p.vsh + t * p.vst) * elem_bytes + 16 * c;
    *(uint4*)(k + kd) = *(const uint4*)(k + ks);
    *(uint4*)(v + vd) = *(const uint4*)(v + vs);
  }
}

}  // namespace

extern "C" {

pa_block_manager* paged_attn_bm_create(int32_t num_blocks, int32_t block_size) {
  if (num_blocks <= 0 || !pow2(block_size) || block_size > 1024) return nullptr;
  pa_block_manager* bm = new (std::nothrow) pa_block_manager;
  if (!bm) return nullptr;
  try {
    bm->num_blocks = num_blocks;
    bm->block_size = block_size;
    bm->ref.assign(num_blocks, 0);
    bm->free_list.resize(num_blocks);
    for (int32_t i = 0; i < num_blocks; ++i) bm->free_list[i] = num_blocks - 1 - i;
  } catch (...) {
    delete bm;
    return nullptr;
  }
  return bm;
}

void paged_attn_bm_destroy(pa_block_manager* bm) { delete bm; }

int paged_attn_bm_allocate_blocks(pa_block_manager* bm, int64_t seq_id, int32_t n) {
  if (!bm) return PA_E_NULL;
  if (n < 0) return PA_E_SHAPE;
  if ((size_t)n > bm->free_list.size()) return PA_E_NOMEM;
  try {
    std::vector<int32_t>& list = bm->seqs[seq_id];
    list.reserve(list.size() + n);
    for (int32_t i = 0; i < n; ++i) list.push_back(bm->take());
  } catch (...) {
    return PA_E_NOMEM;
  }
  return PA_OK;
}

int paged_attn_bm_free_sequence(pa_block_manager* bm, int64_t seq_id) {
  if (!bm) return PA_E_NULL;
  auto it = bm->seqs.find(seq_id);
  if (it == bm->seqs.end()) return PA_E_SEQ;
  for (int32_t b : it->second) bm->drop(b);
  bm->seqs.erase(it);
  return PA_OK;
}

int paged_attn_bm_share_prefix(pa_block_manager* bm, int64_t source, int64_t target,
                               int32_t n_blocks) {
  if (!bm) return PA_E_NULL;
  if (n_blocks < 0) return PA_E_SHAPE;
  auto it = bm->seqs.find(source);
  if (it == bm->seqs.end() || (size_t)n_blocks > it->second.size() || source == target ||
      bm->seqs.count(target))
    return PA_E_SEQ;
  try {
    std::vector<int32_t> prefix(it->second.begin(), it->second.begin() + n_blocks);
    for (int32_t b : prefix) ++bm->ref[b];
    bm->seqs.emplace(target, std::move(prefix));
  } catch (...) {
    return PA_E_NOMEM;
  }
  return PA_OK;
}

int paged_attn_bm_cow_block(pa_block_manager* bm, int64_t seq_id, int32_t block_index,
                            int32_t* src, int32_t* dst) {
  if (!bm || !src || !dst) return PA_E_NULL;
  auto it = bm->seqs.find(seq_id);
  if (it == bm->seqs.end() || block_index < 0 || (size_t)block_index >= it->second.size())
    return PA_E_SEQ;
  int32_t& slot = it->second[block_index];
  *src = *dst = slot;
  if (bm->ref[slot] == 1) return 0;
  if (bm->free_list.empty()) return PA_E_NOMEM;
  const int32_t fresh = bm->take();
  bm->drop(slot);  // still referenced by the other sequences
  *dst = fresh;
  slot = fresh;
  return 1;
}

int paged_attn_bm_append_slot(pa_block_manager* bm, int64_t seq_id, int32_t seq_len, int32_t* src,
                              int32_t* dst) {
  if (!bm || !src || !dst) return PA_E_NULL;
  if (seq_len < 0) return PA_E_SEQ;
  const int32_t idx = seq_len / bm->block_size;
  auto it = bm->seqs.find(seq_id);
  const size_t have = it == bm->seqs.end() ? 0 : it->second.size();
  if ((size_t)idx > have) return PA_E_SEQ;  // a gap before the token's block
  if ((size_t)idx == have) {              // the token starts a new block
    *src = *dst = -1;
    const int rc = paged_attn_bm_allocate_blocks(bm, seq_id, 1);
    if (rc == PA_OK) *src = *dst = bm->seqs[seq_id].back();
    return rc;
  }
  return paged_attn_bm_cow_block(bm, seq_id, idx, src, dst);
}

int paged_attn_bm_num_free(const pa_block_manager* bm) {
  return bm ? (int)bm->free_list.size() : PA_E_NULL;
}

int paged_attn_bm_ref_count(const pa_block_manager* bm, int32_t block) {
  if (!bm) return PA_E_NULL;
  if (block < 0 || block >= bm->num_blocks) return PA_E_SEQ;
  return bm->ref[block];
}

int paged_attn_bm_sequence_blocks(const pa_block_manager* bm, int64_t seq_id, int32_t* out,
                                  int32_t cap) {
  if (!bm) return PA_E_NULL;
  auto it = bm->seqs.find(seq_id);
  if (it == bm->seqs.end()) return PA_E_SEQ;
  const std::vector<int32_t>& list = it->second;
  if (cap > 0 && !out) return PA_E_NULL;
  for (int32_t i = 0; i < cap && (size_t)i < list.size(); ++i) out[i] = list[i];
  return (int)list.size();
}

int paged_attn_bm_block_table(const pa_block_manager* bm, const int64_t* seq_ids, int32_t batch,
                              int32_t max_blocks_per_seq, int32_t* table) {
  if (!bm) return PA_E_NULL;
  if (batch < 0 || max_blocks_per_seq <= 0) return PA_E_SHAPE;
  if (batch > 0 && (!seq_ids || !table)) return PA_E_NULL;
  for (int32_t b = 0; b < batch; ++b) {  // check first: a failed call writes nothing
    auto it = bm->seqs.find(seq_ids[b]);
    if (it == bm->seqs.end()) return PA_E_SEQ;
    if (it->second.size() > (size_t)max_blocks_per_seq) return PA_E_SHAPE;
  }
  for (int32_t b = 0; b < batch; ++b) {
    const std::vector<int32_t>& list = bm->seqs.find(seq_ids[b])->second;
    int32_t* row = table + (int64_t)b * max_blocks_per_seq;
    for (int32_t j = 0; j < max_blocks_per_seq; ++j) row[j] = (size_t)j < list.size() ? list[j] : -1;
  }
  return PA_OK;
}

int paged_attn_copy_blocks(const pa_desc* desc, void* k_cache, void* v_cache, const int32_t* pairs,
                           int32_t n, int32_t* status, void* stream) {
  const int rc = paged_attn_validate(desc);
  if (rc != PA_OK) return rc;
  if (n < 0) return PA_E_SHAPE;
  if (n == 0) return PA_OK;
  if (!k_cache || !v_cache || !pairs) return PA_E_NULL;
  if (((uintptr_t)k_cache | (uintptr_t)v_cache) & 15) return PA_E_ALIGN;
  pa::Params p = {};
  p.k = k_cache;
  p.v = v_cache;
  p.status = status;
  p.ksb = desc->k_stride_block;
  p.ksh = desc->k_stride_head;
  p.kst = desc->k_stride_token;
  p.vsb = desc->v_stride_block;
  p.vsh = desc->v_stride_head;
  p.vst = desc->v_stride_token;
  if (desc->flags & PA_FLAG_KV_XPACKED) p.kst = p.vst = desc->head_dim;  // dense bs x d tiles
  p.Hkv = desc->num_kv_heads;
  p.D = desc->head_dim;
  p.NB = desc->num_blocks;
  int lg = 0;
  while ((1 << lg) < desc->block_size) ++lg;
  p.bs_log2 = lg;
  const int eb = desc->kv_dtype == PA_DTYPE_F32 ? 4 : 2;
  hipLaunchKernelGGL(copy_blocks_kernel, dim3(n, desc->num_kv_heads), dim3(256), 0,
                     (hipStream_t)stream, p, pairs, eb);
  return hipGetLastError() == hipSuccess ? PA_OK : PA_E_LAUNCH;
}

}  // extern "C"
