// pa_append.hip -- in-place append of the decode step's new K/V token.
//
// The decode kernels of the transformers "Paged attention" page write the new
// token's keys and values into the paged cache before attending: token t of
// sequence b lives in block block_table[b][t / bs] at offset t mod bs, and the
// new token is t = cache_seqlens[b] (decoding path of that page: the next
// token's slot follows the last cached one). One workgroup per sequence copies
// its H_kv rows of d elements with 16-byte stores. A slot beyond
// max_blocks_per_seq * block_size or behind an entry outside [0, NB) is not
// written and is reported in the status word; the attention that follows then
// clamps or skips it the same way. With the x-packed layout the K row goes out
// as 16-byte pieces into its [d/8, bs, 8] tile and the V row element by element
// into its [d, bs] tile.
#include "pa_kernels.h"

namespace pa {
namespace {

__global__ void __launch_bounds__(256)
append_kernel(Params p, const char* k_new, const char* v_new, int elem_bytes) {
  const int b = blockIdx.x;
  const int L = p.seqlens[b];
  const int lmax = p.MBS << p.bs_log2;
  if (L < 0 || L >= lmax) {
    if (threadIdx.x == 0 && p.status) atomicOr(p.status, kStatusBadSeqlen);
    return;
  }
  const int id = p.table[(int64_t)b * p.MBS + (L >> p.bs_log2)];
  if (id < 0 || id >= p.NB) {
    if (threadIdx.x == 0 && p.status) atomicOr(p.status, kStatusBadBlock);
    return;
  }
  const int64_t off = L & ((1 << p.bs_log2) - 1);
  const int vec = p.D * elem_bytes / 16;  // 16-byte pieces per row
  if (p.xpacked) {
    // x-packed K: piece c (dims 8c .. 8c+7) is row c of the head's [d/8, bs, 8]
    // tile; transposed V: dim i of the token is element i * bs + off of [d, bs]
    const int bs = 1 << p.bs_log2;
    for (int i = threadIdx.x; i < p.Hkv * vec; i += blockDim.x) {
      const int hk = i / vec, c = i - hk * vec;
      const int64_t src = ((int64_t)b * p.Hkv + hk) * p.D * 2 + 16 * c;
      const int64_t kd = (id * p.ksb + hk * p.ksh + ((int64_t)c * bs + off) * 8) * 2;
      *(uint4*)((char*)p.k + kd) = *(const uint4*)(k_new + src);
    }
    for (int i = threadIdx.x; i < p.Hkv * p.D; i += blockDim.x) {
      const int hk = i / p.D, e = i - hk * p.D;
      const int64_t vd = id * p.vsb + hk * p.vsh + (int64_t)e * bs + off;
      ((uint16_t*)p.v)[vd] = ((const uint16_t*)v_new)[(int64_t)b * p.Hkv * p.D + i];
    }
    return;
  }
  for (int i = threadIdx.x; i < p.Hkv * vec; i += blockDim.x) {
    const int hk = i / vec, c = i - hk * vec;
    const int64_t src = ((int64_t)b * p.Hkv + hk) * p.D * elem_bytes + 16 * c;
    const int64_t kd = (id * p.ksb + hk * p.ksh + off * p.kst) * elem_bytes + 16 * c;
    const int64_t vd = (id * p.vsb + hk * p.vsh + off * p.vst) * elem_bytes + 16 * c;
    *(uint4*)((char*)p.k + kd) = *(const uint4*)(k_new + src);
    *(uint4*)((char*)p.v + vd) = *(const uint4*)(v_new + src);
  }
}

}  // namespace

hipError_t launch_append(const Params& p, const void* k_new, const void* v_new, int elem_bytes,
                         hipStream_t s) {
  hipLaunchKernelGGL(append_kernel, dim3(p.B), dim3(256), 0, s, p, (const char*)k_new,
                     (const char*)v_new, elem_bytes);
  return hipGetLastError();
}

}  // namespace pa
