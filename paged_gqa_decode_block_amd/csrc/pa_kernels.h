// pa_kernels.h -- internal to the gfx950 library: launch parameters, device
// helpers and the launcher declarations shared by the kernel translation units.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace pa {

// Largest number of physical blocks one partition may span; the partition
// kernels stage that many block ids in LDS.
constexpr int kTableCap = 1024;

struct Params {
  const void* q;            // [B, Hq, D] fp32, or bf16 when qo_bf16
  const void* k;            // pool, element strides below
  const void* v;
  const int32_t* table;     // [B, MBS]
  const int32_t* seqlens;   // [B]
  void* out;                // [B, Hq, D] fp32, or bf16 when qo_bf16
  // grid and VALU kernels: partition states (NULL on the streaming path)
  float* ws_m;              // [B, Hq, pmax]  running max, base-2 units
  float* ws_l;              // [B, Hq, pmax]  sum of 2^(s - m)
  float* ws_acc;            // [B, Hq, pmax, D] unnormalised output
  // streaming kernel only (NULL otherwise): a record per stream and two state
  // slots per wave (the partly covered streams at the ends of its share); with
  // folding, records of the groups' shared-prefix streams follow the B x Hkv
  // records of the sequences' own streams
  int32_t* ws_link;         // [B (+ groups), Hkv, 2] first state's slot, number of waves
                            // (0: written out)
  float* ws_cm;             // [waves, 2, rps] running max, base-2 units
  float* ws_cl;             // [waves, 2, rps] sum of 2^(s - m)
  float* ws_cacc;           // [waves, 2, rps, D] unnormalised output
  // prefix folding on the streaming path (fold = 0: off): sequences
  // fold * i .. fold * i + fold - 1 form group i; its first ws_vlen[(fold + 1) i]
  // tokens, the same physical blocks in every member's table, are read once
  // for all members (their fold x G query heads in the score MFMA's 16
  // columns), and ws_vlen[(fold + 1) i + 1 + m] tokens past them as member m's
  // own stream
  int fold;
  int rps;                  // state rows per slot: G, or fold * G with folding
  int32_t* ws_vlen;         // [groups, fold + 1] token counts of the virtual sequences
  // with folding, the state of a stream that lies inside one wave's share but
  // is not written out (a folded prefix, or a member's stream behind one) goes
  // to the stream's own rows (record x = -1): stream record i, rows i * rps ..
  float* ws_om;             // [B + groups, Hkv, rps]
  float* ws_ol;             // [B + groups, Hkv, rps]
  float* ws_oacc;           // [B + groups, Hkv, rps, D]
  // grid kernel with the merge in its last block (NULL otherwise): arrivals per
  // (sequence, KV head), zero between calls
  int32_t* ws_cnt;          // [B, Hkv]
  int32_t* status;          // optional
  int64_t ksb, ksh, kst;    // K strides (elements)
  int64_t vsb, vsh, vst;    // V strides
  int B, Hq, Hkv, G, D;
  int bs_log2, NB, MBS;
  int part;                 // partition size in tokens
  int pmax;                 // ceil(MBS * bs / part); streaming path: a bound on a
                            // stream's states, used to size the combine's workgroups
  float qscale;             // scale * log2(e): scores are kept in base-2 units
  int cus;                  // compute units of the device (streaming kernel)
  int len_add;              // tokens attended = cache_seqlens[b] + len_add (1 after an append)
  int qo_bf16;              // q and out are bf16 (else fp32)
  int nwaves;               // the streaming kernel's grid (two state slots per wave)
  int xpacked;              // K [NB, Hkv, D/8, bs, 8] and V [NB, Hkv, D, bs] (16-bit):
                            // element (blk, h, t, i) of K at blk*ksb + h*ksh + (i/8)*8*bs
                            // + 8*t + i%8, of V at blk*vsb + h*vsh + i*bs + t
};

enum { kStatusBadBlock = 1, kStatusBadSeqlen = 2 };

// Launchers (each returns the launch error, hipSuccess when enqueued).
hipError_t launch_partition_valu(const Params& p, int dtype, hipStream_t s);
hipError_t launch_partition_mfma(const Params& p, int dtype, hipStream_t s);
hipError_t launch_combine(const Params& p, hipStream_t s);
// Paged varlen prefill: query rows cu_q[b] .. cu_q[b+1]-1 of sequence b (at
// most max_q of them), keys its p.seqlens[b] cached tokens, causal or not;
// 16-bit K/V only. ws: the key split's arrival counters (zero on entry, left
// zero) and half states, of prefill_workspace_bytes(p, dtype, max_q) bytes; NULL runs
// every work item whole.
hipError_t launch_prefill(const Params& p, int dtype, const int32_t* cu_q, int max_q, int causal,
                          void* ws, hipStream_t s);
// Workspace of the prefill's key split for these parameters (p.B, p.Hkv, p.G,
// p.D, p.qo_bf16, p.cus), the K/V dtype and max_q: 0 when no work item is split.
size_t prefill_workspace_bytes(const Params& p, int dtype, int max_q);
// Leading bytes of that workspace (arrival counters) that must be zero.
size_t prefill_workspace_zeroed_bytes(const Params& p, int dtype, int max_q);
// Write each sequence's new K and V rows ([B, H_kv, d], the cache's element
// type) at token cache_seqlens[b] of its paged cache.
hipError_t launch_append(const Params& p, const void* k_new, const void* v_new, int elem_bytes,
                         hipStream_t s);
// Persistent streaming MFMA kernel on a device with p.cus compute units;
// `variant` picks a ring depth / occupancy pair (0 = default), `nt` the
// non-temporal cache policy for K/V loads.
hipError_t launch_partition_stream(const Params& p, int dtype, int variant, bool nt, hipStream_t s);
// Prefix folding: each group's folded prefix and the virtual sequences'
// lengths (p.ws_vlen), before the streaming kernel.
hipError_t launch_fold_scan(const Params& p, hipStream_t s);
bool stream_supports(int dtype, int D, int G, int block_size, int batch);
// Grid of the streaming kernel (one wave per workgroup) for head_dim D, ring
// variant `variant`, `cus` compute units and at most `chunk_bound` 16-token
// chunks of work; the workspace holds one continuation slot per wave.
int stream_grid(int D, int variant, int cus, int64_t chunk_bound);

// Waves of the streaming kernel that take work for n_chunks chunks: the whole
// grid when each gets at least kStreamMinChunks, else fewer, kept a multiple of
// the compute-unit count while there is at least one per unit.
constexpr int kStreamMinChunks = 16;
__host__ __device__ inline int stream_active_waves(int64_t n_chunks, int grid, int cus) {
  int64_t w = n_chunks / kStreamMinChunks;
  if (w >= grid) return grid;
  if (w >= cus) w = w / cus * cus;
  return (int)(w < 1 ? 1 : w);
}
// The same in 32 bits (the kernel's chunk count is below 2^31).
__host__ __device__ inline int stream_active_waves32(int n_chunks, int grid, int cus) {
  int w = n_chunks / kStreamMinChunks;
  if (w >= grid) return grid;
  if (w >= cus) w = w / cus * cus;
  return w < 1 ? 1 : w;
}
bool valu_supports(int dtype, int D, int G);
bool mfma_supports(int dtype, int D, int G);
// Floats of LDS the grid kernel's merged variant has for 2 n_part G + 16 of
// merge state.
int fused_merge_capacity(int D);

#if defined(__HIPCC__)

// ---- device helpers --------------------------------------------------------

__device__ __forceinline__ float exp2_fast(float x) { return __builtin_amdgcn_exp2f(x); }

// Cache length of sequence b, clamped to [0, MBS * bs] (a bad value is reported).
__device__ __forceinline__ int clamped_len(const Params& p, int b, bool report) {
  int L = p.seqlens[b] + p.len_add;
  const int lmax = p.MBS << p.bs_log2;
  if (L < 0 || L > lmax) {
    if (report && p.status) atomicOr(p.status, kStatusBadSeqlen);
    L = L < 0 ? 0 : lmax;
  }
  return L;
}

// q and out in fp32 or bf16 (p.qo_bf16, uniform). bf16 -> fp32 is exact;
// fp32 -> bf16 rounds to nearest even and keeps NaN a NaN.
__device__ __forceinline__ float bf16_to_f32(uint32_t bits16) { return __uint_as_float(bits16 << 16); }
__device__ __forceinline__ uint32_t f32_to_bf16(float f) {
  const uint32_t u = __float_as_uint(f);
  if ((u & 0x7fffffffu) > 0x7f800000u) return (u >> 16) | 0x40u;
  return (u + 0x7fffu + ((u >> 16) & 1u)) >> 16;
}
// q elements idx .. idx + 3 (idx a multiple of 4) as floats; QO: 0 fp32,
// 1 bf16, -1 read p.qo_bf16 at run time. Kernels whose register budget is tight
// take the dtype as a template argument: a run-time branch at the output store
// made the register allocator spill the streaming kernel's ring.
template <int QO = -1>
__device__ __forceinline__ float4 load_q4(const Params& p, int64_t idx) {
  if (QO == 1 || (QO < 0 && p.qo_bf16)) {
    const uint2 u = *(const uint2*)((const uint16_t*)p.q + idx);
    return make_float4(bf16_to_f32(u.x & 0xffffu), bf16_to_f32(u.x >> 16),
                       bf16_to_f32(u.y & 0xffffu), bf16_to_f32(u.y >> 16));
  }
  return *(const float4*)((const float*)p.q + idx);
}
// out elements idx .. idx + 3 (idx a multiple of 4), and a single element.
template <int QO = -1>
__device__ __forceinline__ void store_out4(const Params& p, int64_t idx, float a, float b, float c,
                                           float d) {
  if (QO == 1 || (QO < 0 && p.qo_bf16))
    *(uint2*)((uint16_t*)p.out + idx) =
        make_uint2(f32_to_bf16(a) | (f32_to_bf16(b) << 16), f32_to_bf16(c) | (f32_to_bf16(d) << 16));
  else
    *(float4*)((float*)p.out + idx) = make_float4(a, b, c, d);
}
__device__ __forceinline__ void store_out1(const Params& p, int64_t idx, float v) {
  if (p.qo_bf16)
    ((uint16_t*)p.out)[idx] = (uint16_t)f32_to_bf16(v);
  else
    ((float*)p.out)[idx] = v;
}

// Stage the physical ids of blocks [j0, j1] of sequence b in LDS; an id outside
// [0, NB) becomes -1 (never dereferenced) and is reported.
__device__ __forceinline__ void stage_block_ids(const Params& p, int b, int j0, int j1, int* s_ids,
                                                int tid, int nthreads) {
  const int32_t* row = p.table + (int64_t)b * p.MBS;
  for (int j = j0 + tid; j <= j1; j += nthreads) {
    int id = row[j];
    if (id < 0 || id >= p.NB) {
      if (p.status) atomicOr(p.status, kStatusBadBlock);
      id = -1;
    }
    s_ids[j - j0] = id;
  }
}

#endif  // __HIPCC__

}  // namespace pa
