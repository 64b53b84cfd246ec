// pa_partition_mfma.hip -- split-KV partition kernel on the gfx950 matrix cores.
//
// One wave (64 lanes) per (KV partition p, KV head, sequence b). The partition's
// tokens are visited in chunks of 32; per chunk:
//
//   scores  S^T[token, head] = K[token, :] . Q'[head, :]   two 16x16x32 MFMA tiles
//           (tokens in M, the G query heads of the group in N, padded to 16),
//           K fed to the A operand straight from a 16-byte global load per lane;
//   update  the running max m, sum l and output acc of each head, in base 2
//           (page "v10_triton_paged_gqa", core principle: m_new = max(m, max s),
//           alpha = exp(m - m_new), p = exp(s - m_new), l = alpha l + sum p,
//           acc = alpha acc + p V);
//   output  O^T[dim, head] += V^T[dim, token] . P^T[token, head]   one 16x16x32
//           MFMA per 16 dims, V staged through LDS to put tokens in K.
//
// K and V of the KV head are loaded once per chunk and shared by all G query
// heads of the group (page "Paged Attention Kernel Architecture for BI-V100",
// section 4). Q and P are split into a high and a low 16-bit part (two MFMAs
// each), so the products carry ~16 mantissa bits instead of 8 and the fp32
// accumulation stays within the fp16/bf16-KV tolerance for any score spread.
//
// Partition states go to the workspace (max, sum, unnormalised output; page
// "Paged Attention Kernel Architecture for BI-V100", section 2, level 3), or,
// when the sequence has one partition, the normalised output goes straight to
// out. Tokens at or past L_b and tokens whose table entry is invalid are never
// loaded; their scores are -inf.
//
// x-packed caches (the layout of the same page, section 3: K [blocks, heads,
// d/8, bs, 8], V [blocks, heads, d, bs]): each lane's 16-byte K piece is the
// same fragment as before, read from its row of the packed tile; V arrives as
// V^T, 8 consecutive tokens of one dim per 16-byte read, is staged as V^T rows
// and gives the P . V operand by plain 8-byte LDS reads (no transposing read).
//
// Merged variant (one launch): the same page, section 2, lets the last
// partition block to finish do the merge instead of a second kernel. Every
// block of a multi-partition sequence publishes its state with write-through
// stores that are coherent across the device's L2 caches, waits for them to
// complete, and counts itself in on a per-(sequence, KV head) arrival word. The
// block that arrives last resets the word to zero for the next call and folds
// the G x n_part states with the max-rescaling combine, reading them with loads
// that see the other L2s' writes (no cache write-back or invalidate is needed).
// One wave reads all of a KV head's states, so this pays off for short
// contexts (few partitions) and loses to the separate combine kernel for long
// ones.
#include "pa_kernels.h"

namespace pa {
namespace {

typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));
typedef uint16_t u16x8 __attribute__((ext_vector_type(8)));

template <typename T>
struct Mma;

template <>
struct Mma<__bf16> {
  typedef bf16x8 vec;
  static __device__ __forceinline__ f32x4 mma(vec a, vec b, f32x4 c) {
    return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
  }
};

template <>
struct Mma<_Float16> {
  typedef f16x8 vec;
  static __device__ __forceinline__ f32x4 mma(vec a, vec b, f32x4 c) {
    return __builtin_amdgcn_mfma_f32_16x16x32_f16(a, b, c, 0, 0, 0);
  }
};

// Split x into hi + lo, both rounded to T (round to nearest even).
template <typename T>
__device__ __forceinline__ void split2(float x, T& hi, T& lo) {
  hi = (T)x;
  lo = (T)(x - (float)hi);
}

// LDS layout of the V chunk: 32 token rows of D elements, row-major, with the
// 16-byte column chunks of row R XOR-permuted by f(R) = 2*(R&3) + ((R>>2)&1).
// Each group of 8 lanes writing 16-byte chunks of rows 0..7 (or 8..15) then hits
// 8 different bank groups, and so do the 16 lanes of a quad in the transposing
// reads below.
__device__ __forceinline__ int vswz(int R) { return ((R & 3) << 1) | ((R >> 2) & 1); }

typedef short s16x4 __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) s16x4 lds_s16x4;


// Cache-coherence bits of the merged variant's workspace traffic: SC1 set,
// SC0 clear is device scope on gfx950 (the ISA's SC1:SC0 scope field: wave,
// group, device, system). A device-scope store is written through the XCD's
// L2 to the device-coherent level, and the wave's vector-memory counter drops
// for it only once it is complete there; a device-scope load is served from
// that level, not from a line another XCD's write left stale in this XCD's L2.
constexpr int kSc1 = 16;
typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));

// Raw buffer descriptor over [ptr, ptr + bytes) (uniform across the wave); an
// offset at or past `bytes` loads zeros and stores nothing.
__device__ __forceinline__ __amdgpu_buffer_rsrc_t ws_rsrc(const void* ptr, int bytes) {
  const uint64_t a = (uint64_t)ptr;
  const uint32_t lo = __builtin_amdgcn_readfirstlane((int)(uint32_t)a);
  const uint32_t hi = __builtin_amdgcn_readfirstlane((int)(uint32_t)(a >> 32));
  return __builtin_amdgcn_make_buffer_rsrc((void*)(((uint64_t)hi << 32) | lo), (short)0,
                                           __builtin_amdgcn_readfirstlane(bytes), 0x00020000);
}

// Merged variant, after the partition loop of partition `part` of
// (sequence b, KV head hk): publish this block's states (lane (q, r): head r,
// dims 16 mb + 4 q .. +3), count in, and if this block is the last of the
// n_part to arrive, write out = sum_p w_p acc_p / sum_p w_p l_p with
// w_p = 2^(m_p - max_p m_p) for the G heads. s_f: 16 D floats of LDS, at least
// 2 n_part G + 16 of them (checked on the host).
template <int D>
__device__ __forceinline__ void publish_and_merge(const Params& p, int b, int hk, int part,
                                                  int npart, const f32x4 (&acc)[D / 16], float m,
                                                  float l, float* s_f) {
  constexpr int MB = D / 16;
  const int lane = threadIdx.x, r = lane & 15, q = lane >> 4;
  const int G = p.G, pm = p.pmax;
  // the KV head's states: head g, partition i at row g * pmax + i
  const int64_t row0 = ((int64_t)b * p.Hq + (int64_t)hk * G) * pm;
  const int nacc = G * pm * D * 4;
  const __amdgpu_buffer_rsrc_t racc = ws_rsrc(p.ws_acc + row0 * D, nacc);
  const __amdgpu_buffer_rsrc_t rm = ws_rsrc(p.ws_m + row0, G * pm * 4);
  const __amdgpu_buffer_rsrc_t rl = ws_rsrc(p.ws_l + row0, G * pm * 4);
  if (r < G) {
    const int o = ((r * pm + part) * D + 4 * q) * 4;
#pragma unroll
    for (int mb = 0; mb < MB; ++mb)
      __builtin_amdgcn_raw_buffer_store_b128(__builtin_bit_cast(u32x4, acc[mb]), racc, o + 64 * mb,
                                             0, kSc1);
    if (q == 0) {
      __builtin_amdgcn_raw_buffer_store_b32(__float_as_uint(m), rm, (r * pm + part) * 4, 0, kSc1);
      __builtin_amdgcn_raw_buffer_store_b32(__float_as_uint(l), rl, (r * pm + part) * 4, 0, kSc1);
    }
  }
  // Ordering of the states against the arrival counter, by the device-scope
  // cache bits above rather than by C++ release / acquire fences (which
  // compile to a write-back and an invalidate of the whole L2 of the XCD, and
  // made this variant 33-51 % slower on the 64-sequence and prefix-shared
  // batches):
  //  1. every state store above is device scope, so it completes only at the
  //     device-coherent level;
  //  2. s_waitcnt(0) waits until all of this wave's stores are complete before
  //     the increment is issued (the signal fences keep the compiler from
  //     moving memory operations across the wait);
  //  3. the increment is an agent-scope atomic read-modify-write, so the
  //     n_part increments of the counter happen one after another in a single
  //     order at the device's point of coherence for it; the block that reads
  //     n_part - 1 executes its increment after every other block's, and each
  //     of those was issued only after that block's stores were complete;
  //  4. that block's loads below are issued after its increment returned (they
  //     depend on its value through the branch) and are device scope too, so
  //     they read the completed states and no stale L2 line.
  // The same device-scope bits are how agent-scope atomic loads and stores
  // are made coherent on this target family.
  __atomic_signal_fence(__ATOMIC_SEQ_CST);
  __builtin_amdgcn_s_waitcnt(0);
  __atomic_signal_fence(__ATOMIC_SEQ_CST);
  int32_t* cnt = p.ws_cnt + (b * p.Hkv + hk);
  int prev = 0;
  if (lane == 0) prev = __hip_atomic_fetch_add(cnt, 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  prev = __builtin_amdgcn_readfirstlane(prev);
  if (prev != npart - 1) return;
  // last to arrive: reset the counter for the next call (the kernel boundary
  // orders this store before any later launch)
  if (lane == 0) __hip_atomic_store(cnt, 0, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  __atomic_signal_fence(__ATOMIC_SEQ_CST);

  // Pass 1, lane (q, r) for head r: m and l of partitions i = q (mod 4) into
  // LDS (16 per lane per round, loads in flight together), the head's max.
  float* s_m = s_f;             // [n_part][G], then the weights w
  float* s_l = s_f + npart * G;  // [n_part][G]
  float* s_L = s_l + npart * G;  // [G] sum_p w_p l_p
  float mx = -INFINITY;
  for (int i0 = 0; i0 < npart; i0 += 64) {
    float mv[16], lv[16];
#pragma unroll
    for (int k = 0; k < 16; ++k) {
      const int i = i0 + 4 * k + q;
      const int o = (r < G && i < npart) ? (r * pm + i) * 4 : G * pm * 4;  // past the end: 0
      mv[k] = __uint_as_float(__builtin_amdgcn_raw_buffer_load_b32(rm, o, 0, kSc1));
      lv[k] = __uint_as_float(__builtin_amdgcn_raw_buffer_load_b32(rl, o, 0, kSc1));
    }
#pragma unroll
    for (int k = 0; k < 16; ++k) {
      const int i = i0 + 4 * k + q;
      if (r < G && i < npart) {
        s_m[i * G + r] = mv[k];
        s_l[i * G + r] = lv[k];
        mx = fmaxf(mx, mv[k]);
      }
    }
  }
  mx = fmaxf(mx, __shfl_xor(mx, 16));
  mx = fmaxf(mx, __shfl_xor(mx, 32));
  const float mu = mx == -INFINITY ? 0.f : mx;
  float ls = 0.f;
  if (r < G) {
    for (int i = q; i < npart; i += 4) {
      const float w = exp2_fast(s_m[i * G + r] - mu);
      s_m[i * G + r] = w;
      ls += w * s_l[i * G + r];
    }
  }
  ls += __shfl_xor(ls, 16);
  ls += __shfl_xor(ls, 32);
  if (r < G && q == 0) s_L[r] = ls;
  __syncthreads();

  // Pass 2: slot s = (head s / (D/4), dims 4 (s % (D/4)) .. +3); each lane
  // folds 4 slots over 8 partitions per round (32 16-byte loads in flight).
  constexpr int SPH = D / 4;  // slots per head
  const int nslot = G * SPH;
  for (int s0 = 0; s0 < nslot; s0 += 4 * 64) {
    int hs[4], ob[4];
    bool sv[4];
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      const int sl = s0 + 64 * u + lane;
      sv[u] = sl < nslot;
      hs[u] = sv[u] ? sl / SPH : 0;
      ob[u] = (hs[u] * pm * D + 4 * (sl % SPH)) * 4;
    }
    float4 a[4];
#pragma unroll
    for (int u = 0; u < 4; ++u) a[u] = make_float4(0.f, 0.f, 0.f, 0.f);
    for (int i0 = 0; i0 < npart; i0 += 8) {
      u32x4 x[4][8];
#pragma unroll
      for (int u = 0; u < 4; ++u)
#pragma unroll
        for (int k = 0; k < 8; ++k) {
          const int i = i0 + k;
          const int o = (sv[u] && i < npart) ? ob[u] + i * D * 4 : nacc;  // past the end: 0
          x[u][k] = __builtin_amdgcn_raw_buffer_load_b128(racc, o, 0, kSc1);
        }
#pragma unroll
      for (int u = 0; u < 4; ++u)
#pragma unroll
        for (int k = 0; k < 8; ++k) {
          // a partition past n_part loaded zeros; its (clamped) weight is finite
          const float w = s_m[min(i0 + k, npart - 1) * G + hs[u]];
          a[u].x += w * __uint_as_float(x[u][k][0]);
          a[u].y += w * __uint_as_float(x[u][k][1]);
          a[u].z += w * __uint_as_float(x[u][k][2]);
          a[u].w += w * __uint_as_float(x[u][k][3]);
        }
    }
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      if (!sv[u]) continue;
      const float tot = s_L[hs[u]];
      const float inv = tot > 0.f ? 1.f / tot : 0.f;
      const int sl = s0 + 64 * u + lane;
      store_out4(p, ((int64_t)b * p.Hq + hk * G + hs[u]) * D + 4 * (sl % SPH), a[u].x * inv,
                 a[u].y * inv, a[u].z * inv, a[u].w * inv);
    }
  }
}

// Waves per SIMD the register allocation is held to: 2 for d <= 128, 1 for d = 256.
template <int D>
struct Occ {
  static constexpr int waves = D <= 128 ? 2 : 1;
};

template <typename T, int D, bool FUSED, bool XP>
__global__ void __launch_bounds__(64) __attribute__((amdgpu_waves_per_eu(Occ<D>::waves)))
partition_mfma_kernel(Params p) {
  typedef typename Mma<T>::vec V8;
  constexpr int KS = D / 32;  // k-steps of a 16-token score tile
  constexpr int MB = D / 16;  // 16-dim output tiles
  constexpr bool kQInLds = D > 128;  // Q' fragments: LDS for d = 256, registers otherwise
  // V register sets: two (refill distance 64 tokens) for d <= 128; one for d = 256
  // and for the x-packed layout (whose V^T addressing needs more registers),
  // refilled with the next chunk as soon as it is staged in LDS.
  constexpr int kVDist = (D > 128 || XP) ? 32 : 64;

  __shared__ int s_ids[kTableCap];
  __shared__ __attribute__((aligned(16))) uint16_t s_v[32 * D];
  __shared__ __attribute__((aligned(16))) V8 s_q[kQInLds ? 2 : 1][kQInLds ? KS : 1][64];

  // Partition-major grid: x = b * H_kv + hk, y = partition. Consecutive
  // workgroup ids (which the dispatcher deals round-robin to the XCDs) cover all
  // (sequence, KV head) pairs of one partition index.
  const int b = blockIdx.x / p.Hkv, hk = blockIdx.x - (blockIdx.x / p.Hkv) * p.Hkv;
  const int part = blockIdx.y;
  const int lane = threadIdx.x;
  const int r = lane & 15, q = lane >> 4;
  const int G = p.G;

  const int L = clamped_len(p, b, part == 0 && hk == 0 && lane == 0);
  if (L == 0) {
    if (part == 0) {  // empty context: zeros
      for (int i = lane; i < G * D / 4; i += 64) {
        const int g = i / (D / 4), c4 = i % (D / 4);
        store_out4(p, ((int64_t)b * p.Hq + hk * G + g) * D + 4 * c4, 0.f, 0.f, 0.f, 0.f);
      }
    }
    return;
  }
  const int npart = (L + p.part - 1) / p.part;
  if (part >= npart) return;
  const int t0 = part * p.part;
  const int t1 = min(L, t0 + p.part);
  const int bsm = (1 << p.bs_log2) - 1;
  const int j0 = t0 >> p.bs_log2;
  stage_block_ids(p, b, j0, (t1 - 1) >> p.bs_log2, s_ids, lane, 64);

  // Q' = q * scale * log2(e) of head r of the group (zero for padded heads),
  // dims 32*ks + 8*q .. +7: the B-operand fragments of the score MFMAs, split
  // into hi / lo parts.
  V8 qreg[kQInLds ? 1 : 2][kQInLds ? 1 : KS];
  {
    const bool hv = r < G;
    const int64_t qrow = ((int64_t)b * p.Hq + hk * G + (hv ? r : 0)) * D + 8 * q;
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) {
      float4 a = hv ? load_q4(p, qrow + 32 * ks) : make_float4(0, 0, 0, 0);
      float4 c = hv ? load_q4(p, qrow + 32 * ks + 4) : make_float4(0, 0, 0, 0);
      const float x[8] = {a.x, a.y, a.z, a.w, c.x, c.y, c.z, c.w};
      V8 hi, lo;
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        T h, l2;
        split2<T>(x[e] * p.qscale, h, l2);
        hi[e] = h;
        lo[e] = l2;
      }
      if constexpr (kQInLds) {
        s_q[0][ks][lane] = hi;
        s_q[1][ks][lane] = lo;
      } else {
        qreg[0][ks] = hi;
        qreg[1][ks] = lo;
      }
    }
  }
  __syncthreads();

  // K: lane quad q reads dims 32 ks + 8 q .. +7 of a token. Default layouts:
  // token rows of d elements (stride kst). x-packed: 16-byte piece 4 ks + q of
  // the token is row 4 ks + q of the [d/8, bs, 8] tile (8 elements per token).
  const int bs = 1 << p.bs_log2;
  const T* kbase = (const T*)p.k + (int64_t)hk * p.ksh + (XP ? (int64_t)8 * bs * q : 8 * q);
  const int64_t kks = XP ? (int64_t)32 * bs : 32;  // elements from dims 32 ks to 32 (ks + 1)
  const int64_t kst = XP ? 8 : p.kst;
  const T* vbase = (const T*)p.v + (int64_t)hk * p.vsh + (XP ? 0 : 8 * q);

  f32x4 acc[MB];
#pragma unroll
  for (int i = 0; i < MB; ++i) acc[i] = f32x4{0.f, 0.f, 0.f, 0.f};
  float m = -INFINITY, l = 0.f;

  // K or V of chunk c: lane (q, r) takes token c + 16*tau + r, dims
  // 32*ks + 8*q .. +7 (for K exactly the A-operand fragment of the score MFMA).
  // Tokens at or past t1, or behind an invalid table entry, are not loaded.
  auto load_rows = [&](int c, const T* base, int64_t sblk, int64_t stok, int64_t sks,
                       uint4 (&dst)[2][KS], bool (&ok)[2]) {
#pragma unroll
    for (int tau = 0; tau < 2; ++tau) {
      const int t = c + 16 * tau + r;
      const int id = t < t1 ? s_ids[(t >> p.bs_log2) - j0] : -1;
      ok[tau] = id >= 0;
#pragma unroll
      for (int ks = 0; ks < KS; ++ks) dst[tau][ks] = make_uint4(0, 0, 0, 0);
      if (id >= 0) {
        const T* src = base + (int64_t)id * sblk + (int64_t)(t & bsm) * stok;
#pragma unroll
        for (int ks = 0; ks < KS; ++ks) dst[tau][ks] = *(const uint4*)(src + sks * ks);
      }
    }
  };

  // x-packed layout, V of chunk c from its [d, bs] tiles: piece j of the lane
  // (pc = lane + 64 j) is dim pc / 4, tokens c + 8 (pc % 4) .. +7, 16 bytes of
  // one block (bs >= 8). The piece holding t1 - 1 is read element by element up
  // to it; pieces at or past t1 or behind an invalid entry are not read.
  auto load_vt = [&](int c, uint4 (&dst)[2][KS]) {
    // every piece of the lane has the same tokens (pc % 4 = lane % 4): one
    // table lookup and one base address; piece j is 16 dims further
    const int t = c + 8 * (lane & 3);
    const int id = t < t1 ? s_ids[(t >> p.bs_log2) - j0] : -1;
    const T* src = vbase + (int64_t)(id < 0 ? 0 : id) * p.vsb + (int64_t)(lane >> 2) * bs + (t & bsm);
    const bool full = id >= 0 && t + 8 <= t1;
    const bool tail = id >= 0 && t + 8 > t1;
#pragma unroll
    for (int tau = 0; tau < 2; ++tau) {
#pragma unroll
      for (int ks = 0; ks < KS; ++ks) {
        const T* sp = src + (int64_t)16 * bs * (tau * KS + ks);
        uint4 x = make_uint4(0, 0, 0, 0);
        if (full) {
          x = *(const uint4*)sp;
        } else if (tail) {
          uint32_t e[8];
#pragma unroll
          for (int i = 0; i < 8; ++i) e[i] = t + i < t1 ? ((const uint16_t*)sp)[i] : 0u;
          x = make_uint4(e[0] | (e[1] << 16), e[2] | (e[3] << 16), e[4] | (e[5] << 16),
                         e[6] | (e[7] << 16));
        }
        dst[tau][ks] = x;
      }
    }
  };
  // x-packed V^T tile in LDS: row d (a dim) holds the chunk's 32 tokens as four
  // 16-byte octets, octet o stored at o ^ ((d >> 2) & 3), so that both the
  // staging writes and the 8-byte fragment reads of 16 consecutive dims spread
  // over all banks.
  auto vt_slot = [](int d, int o) { return d * 32 + 8 * (o ^ ((d >> 2) & 3)); };

  // Per-lane pieces of the transposing V reads: lane (q, 4j + k) points at row
  // 16*tau + 4q + j, columns 16*mb + 4k .. +3.
  const int tj = r >> 2, tk = r & 3;
  const int trow = (4 * q + tj) * D + 4 * (tk & 1);
  const int txor = (tk >> 1) ^ (q & 1);

  // One 32-token chunk. kr/okr hold its K, vr its V; the K set is refilled with
  // chunk c + 64 once the scores are formed and the V set with chunk
  // c + kVDist once it is staged, so about two chunks of loads stay in flight
  // behind the compute.
  auto step = [&](int c, uint4 (&kr)[2][KS], bool (&okr)[2], uint4 (&vr)[2][KS]) {
    const bool refill = c + 64 < t1;
    // ---- stage V in LDS (row-major, swizzled; x-packed: V^T rows), then refill vr
    if constexpr (XP) {
#pragma unroll
      for (int tau = 0; tau < 2; ++tau)
#pragma unroll
        for (int ks = 0; ks < KS; ++ks) {
          const int pc = lane + 64 * (tau * KS + ks);
          *(uint4*)(s_v + vt_slot(pc >> 2, pc & 3)) = vr[tau][ks];
        }
      if (c + kVDist < t1) load_vt(c + kVDist, vr);
    } else {
#pragma unroll
      for (int tau = 0; tau < 2; ++tau) {
        const int R = 16 * tau + r;
        const int f = vswz(R);
#pragma unroll
        for (int ks = 0; ks < KS; ++ks)
          *(uint4*)(s_v + R * D + 8 * ((4 * ks + q) ^ f)) = vr[tau][ks];
      }
      bool dummy[2];
      if (c + kVDist < t1) load_rows(c + kVDist, vbase, p.vsb, p.vst, 32, vr, dummy);
    }

    // ---- scores: two 16-token tiles, K . Q'hi + K . Q'lo
    f32x4 st[2] = {f32x4{0.f, 0.f, 0.f, 0.f}, f32x4{0.f, 0.f, 0.f, 0.f}};
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) {
      V8 qh, ql;
      if constexpr (kQInLds) {
        qh = s_q[0][ks][lane];
        ql = s_q[1][ks][lane];
      } else {
        qh = qreg[0][ks];
        ql = qreg[1][ks];
      }
#pragma unroll
      for (int tau = 0; tau < 2; ++tau) {
        const V8 a = __builtin_bit_cast(V8, kr[tau][ks]);
        st[tau] = Mma<T>::mma(a, qh, st[tau]);
        st[tau] = Mma<T>::mma(a, ql, st[tau]);
      }
    }
    // token 16*tau + x was loaded iff lane x (quad 0) had a valid id for it
    const uint64_t bal0 = __ballot(okr[0]);
    const uint64_t bal1 = __ballot(okr[1]);
    if (refill) load_rows(c + 64, kbase, p.ksb, kst, kks, kr, okr);

    float sv[8];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      sv[i] = ((bal0 >> (4 * q + i)) & 1) ? st[0][i] : -INFINITY;
      sv[4 + i] = ((bal1 >> (4 * q + i)) & 1) ? st[1][i] : -INFINITY;
    }

    // ---- running softmax state of head r (same in all four quads)
    float mt = sv[0];
#pragma unroll
    for (int i = 1; i < 8; ++i) mt = fmaxf(mt, sv[i]);
    mt = fmaxf(mt, __shfl_xor(mt, 16));
    mt = fmaxf(mt, __shfl_xor(mt, 32));
    const float mn = fmaxf(m, mt);
    const float mu = mn == -INFINITY ? 0.f : mn;
    const float alpha = exp2_fast(m - mu);
    float pv[8], ps = 0.f;
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      pv[i] = exp2_fast(sv[i] - mu);
      ps += pv[i];
    }
    l = l * alpha + ps;
    m = mn;
#pragma unroll
    for (int i = 0; i < MB; ++i) acc[i] *= alpha;

    // P^T fragment: k-slot j holds token 16*(j>>2) + 4*q + (j&3)
    V8 phi, plo;
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      T h, lo;
      split2<T>(pv[j], h, lo);
      phi[j] = h;
      plo[j] = lo;
    }

    // ---- O^T += V^T P^T: the V^T fragment of slots j = 0..3 / 4..7 comes from
    // one transposing 64-bit LDS read each (16-lane group semantics: lane i gets
    // element i%4 of the 8 bytes addressed by lane 4j + i/4, for j = 0..3).
#pragma unroll
    for (int mb = 0; mb < MB; ++mb) {
      s16x4 lo4, hi4;
      if constexpr (XP) {
        // slots 0..3: tokens 4q .. 4q+3 (octet q / 2), 4..7: 16 + 4q .. (octet 2 + q / 2)
        const int d = 16 * mb + r;
        lo4 = *(const s16x4*)(s_v + vt_slot(d, q >> 1) + 4 * (q & 1));
        hi4 = *(const s16x4*)(s_v + vt_slot(d, 2 + (q >> 1)) + 4 * (q & 1));
      } else {
        const int pc = 2 * (mb ^ tj) + txor;
        lo4 = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4*)(s_v + trow + 8 * pc));
        hi4 = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4*)(s_v + 16 * D + trow + 8 * pc));
      }
      const V8 av = __builtin_bit_cast(V8, __builtin_shufflevector(lo4, hi4, 0, 1, 2, 3, 4, 5, 6, 7));
      acc[mb] = Mma<T>::mma(av, phi, acc[mb]);
      acc[mb] = Mma<T>::mma(av, plo, acc[mb]);
    }
  };

  uint4 kA[2][KS], kB[2][KS], vA[2][KS], vB[kVDist == 64 ? 2 : 1][KS];
  bool okA[2], okB[2] = {false, false};
  if constexpr (XP)
    load_vt(t0, vA);
  else
    load_rows(t0, vbase, p.vsb, p.vst, 32, vA, okA);
  load_rows(t0, kbase, p.ksb, kst, kks, kA, okA);
  if (t0 + 32 < t1) {
    if constexpr (kVDist == 64) {
      if constexpr (XP)
        load_vt(t0 + 32, vB);
      else
        load_rows(t0 + 32, vbase, p.vsb, p.vst, 32, vB, okB);
    }
    load_rows(t0 + 32, kbase, p.ksb, kst, kks, kB, okB);
  }
  for (int c = t0; c < t1; c += 64) {
    step(c, kA, okA, vA);
    if (c + 32 >= t1) break;
    if constexpr (kVDist == 64)
      step(c + 32, kB, okB, vB);
    else
      step(c + 32, kB, okB, vA);
  }

  // l summed over the four quads (each holds its own tokens' share)
  l += __shfl_xor(l, 16);
  l += __shfl_xor(l, 32);

  if constexpr (FUSED) {
    if (npart > 1) {
      __syncthreads();  // the V tile's LDS is reused by the merge
      publish_and_merge<D>(p, b, hk, part, npart, acc, m, l, (float*)s_v);
      return;
    }
  }
  if (r >= G) return;
  const int h = hk * G + r;
  if (npart == 1) {
    const float inv = l > 0.f ? 1.f / l : 0.f;
    const int64_t orow = ((int64_t)b * p.Hq + h) * D + 4 * q;
#pragma unroll
    for (int mb = 0; mb < MB; ++mb) {
      const f32x4 o = acc[mb] * inv;
      store_out4(p, orow + 16 * mb, o[0], o[1], o[2], o[3]);
    }
  } else {
    const int64_t row = ((int64_t)b * p.Hq + h) * p.pmax + part;
    float* ap = p.ws_acc + row * D + 4 * q;
#pragma unroll
    for (int mb = 0; mb < MB; ++mb)
      *(float4*)(ap + 16 * mb) = make_float4(acc[mb][0], acc[mb][1], acc[mb][2], acc[mb][3]);
    if (q == 0) {
      p.ws_m[row] = m;
      p.ws_l[row] = l;
    }
  }
}

template <typename T, int D>
hipError_t launch_t(const Params& p, hipStream_t s) {
  dim3 grid(p.B * p.Hkv, p.pmax);
  if (p.xpacked) {
    if (p.ws_cnt)
      hipLaunchKernelGGL((partition_mfma_kernel<T, D, true, true>), grid, dim3(64), 0, s, p);
    else
      hipLaunchKernelGGL((partition_mfma_kernel<T, D, false, true>), grid, dim3(64), 0, s, p);
  } else if (p.ws_cnt) {
    hipLaunchKernelGGL((partition_mfma_kernel<T, D, true, false>), grid, dim3(64), 0, s, p);
  } else {
    hipLaunchKernelGGL((partition_mfma_kernel<T, D, false, false>), grid, dim3(64), 0, s, p);
  }
  return hipGetLastError();
}

template <typename T>
hipError_t launch_d(const Params& p, hipStream_t s) {
  switch (p.D) {
    case 64: return launch_t<T, 64>(p, s);
    case 128: return launch_t<T, 128>(p, s);
    case 256: return launch_t<T, 256>(p, s);
  }
  return hipErrorInvalidValue;
}

}  // namespace

int fused_merge_capacity(int D) { return 16 * D; }

bool mfma_supports(int dtype, int D, int G) {
  return (dtype == 1 || dtype == 2) && (D == 64 || D == 128 || D == 256) && G >= 1 && G <= 16;
}

hipError_t launch_partition_mfma(const Params& p, int dtype, hipStream_t s) {
  if (dtype == 1) return launch_d<_Float16>(p, s);
  if (dtype == 2) return launch_d<__bf16>(p, s);
  return hipErrorInvalidValue;
}

}  // namespace pa
