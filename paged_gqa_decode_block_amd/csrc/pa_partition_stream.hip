// pa_partition_stream.hip -- persistent streaming partition kernel (MFMA, gfx950).
//
// The work items are the (sequence b, KV head, KV partition p) triples of the
// split-KV decomposition (page "Paged Attention Kernel Architecture for
// BI-V100", sections 4 and 6), numbered sequence by sequence, KV head by KV
// head, partition by partition. One wave per SIMD is launched and wave w takes a
// contiguous run of items, so it mostly walks one (b, KV head) token stream
// across several partitions. Along that stream it keeps a ring of NBUF 16-token
// chunks of K and V in flight in registers (as many as the 6-bit vector-memory
// counter can track), so the memory system always has ~50-60 KB per wave
// outstanding and no partition starts with an empty pipeline.
//
// Loads are raw buffer loads of full token rows (each 16-byte lane load is part
// of a contiguous row segment of 128-512 bytes) with the non-temporal hint. The
// per-chunk buffer descriptor (built in scalar registers) starts at the chunk's
// first row and its size covers only the attended rows, so rows past L_b and
// chunks behind an invalid table entry read as zeros without touching memory.
// Each chunk is then written to two swizzled LDS tiles and read back in MFMA
// operand layout:
//
//   scores  S^T[token, head] = K[token, :] . Q'[head, :]      16x16x32 MFMAs
//           (16 tokens in M, the group's G query heads in N, padded to 16)
//   update  running max m, sum l and unnormalised output per head, in base 2
//           (page "v10_triton_paged_gqa", core principle)
//   output  O^T[dim, head] += V^T[dim, token] . P^T[token, head]  16x16x16
//           MFMAs; the V^T fragment is one transposing 64-bit LDS read and the
//           P^T fragment is the score MFMA's own output layout.
//
// Q' and P are split into hi + lo 16-bit parts (two MFMAs each) so products keep
// ~16 mantissa bits. The running output is rescaled lazily: p = 2^(s - m) uses a
// reference max m that is only raised (and acc, l rescaled) when a score exceeds
// it by more than 8, so p <= 256 and most chunks skip the rescale. Whenever the stream crosses a partition boundary the
// partition's state is written (workspace, or normalised output when the
// sequence has one partition) and reset. Tokens at or past L_b and chunks behind
// an invalid table entry are never loaded; their scores are -inf.
//
// Requires block_size >= 16 (a 16-token chunk lies in one block) and at most
// 1024 sequences (the item prefix is formed in registers).
#include <type_traits>

#include "pa_kernels.h"

namespace pa {
namespace {

// Compile-time loop: f(integral_constant<int, I>) for I in [I0, N).
template <int I, int N, typename F>
__device__ __forceinline__ void static_for(F&& f) {
  if constexpr (I < N) {
    f(std::integral_constant<int, I>{});
    static_for<I + 1, N>(f);
  }
}

typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));
typedef short s16x4 __attribute__((ext_vector_type(4)));
typedef _Float16 f16x4 __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) s16x4 lds_s16x4;

constexpr int kMaxWindows = 16;  // 16 x 64 = 1024 sequences

template <typename T>
struct Mx;

template <>
struct Mx<__bf16> {
  typedef bf16x8 v8;
  typedef s16x4 v4;
  static __device__ __forceinline__ f32x4 mma32(v8 a, v8 b, f32x4 c) {
    return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
  }
  static __device__ __forceinline__ f32x4 mma16(v4 a, v4 b, f32x4 c) {
    return __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(a, b, c, 0, 0, 0);
  }
  static __device__ __forceinline__ v4 pack(bf16x4 x) { return __builtin_bit_cast(v4, x); }
  typedef bf16x4 e4;
};

template <>
struct Mx<_Float16> {
  typedef f16x8 v8;
  typedef f16x4 v4;
  static __device__ __forceinline__ f32x4 mma32(v8 a, v8 b, f32x4 c) {
    return __builtin_amdgcn_mfma_f32_16x16x32_f16(a, b, c, 0, 0, 0);
  }
  static __device__ __forceinline__ f32x4 mma16(v4 a, v4 b, f32x4 c) {
    return __builtin_amdgcn_mfma_f32_16x16x16f16(a, b, c, 0, 0, 0);
  }
  static __device__ __forceinline__ v4 pack(f16x4 x) { return x; }
  typedef f16x4 e4;
};

template <int D>
struct Cfg {
  static constexpr int CPR = D / 8;         // 16-byte chunks per token row
  static constexpr int RPI = 64 / CPR;      // token rows per load instruction (8, 4, 2)
  static constexpr int LPC = 16 / RPI;      // load instructions per 16-token chunk (2, 4, 8)
  static constexpr int KS = D / 32;         // k-steps of the score MFMA
  static constexpr int MB = D / 16;         // 16-dim output tiles
};

// Raw buffer descriptor word 3 for plain 32-bit data on gfx950.
constexpr int kRsrcWord3 = 0x00020000;
// Raw buffer descriptor over [ptr, ptr + bytes); ptr and bytes are the same in
// every lane, which readfirstlane makes visible to the compiler (no waterfall).
__device__ __forceinline__ __amdgpu_buffer_rsrc_t uniform_rsrc(const char* ptr, int bytes) {
  const uint64_t a = (uint64_t)ptr;
  const uint32_t lo = __builtin_amdgcn_readfirstlane((int)(uint32_t)a);
  const uint32_t hi = __builtin_amdgcn_readfirstlane((int)(uint32_t)(a >> 32));
  const int n = __builtin_amdgcn_readfirstlane(bytes);
  return __builtin_amdgcn_make_buffer_rsrc((void*)(((uint64_t)hi << 32) | lo), (short)0, n, kRsrcWord3);
}

// POL: cache policy bits of the K/V loads (0 = default, 2 = non-temporal).
template <int POL>
__device__ __forceinline__ uint4 buf_load(__amdgpu_buffer_rsrc_t r, int voff) {
  const u32x4 t = __builtin_amdgcn_raw_buffer_load_b128(r, voff, 0, POL);
  return make_uint4(t[0], t[1], t[2], t[3]);
}

// Max / sum over the four 16-lane quads (lanes i, i^16, i^32, i^48).
__device__ __forceinline__ float quad_max(float x) {
  auto a = __builtin_amdgcn_permlane16_swap(__builtin_bit_cast(int, x), __builtin_bit_cast(int, x),
                                            false, false);
  x = fmaxf(__builtin_bit_cast(float, (int)a[0]), __builtin_bit_cast(float, (int)a[1]));
  auto c = __builtin_amdgcn_permlane32_swap(__builtin_bit_cast(int, x), __builtin_bit_cast(int, x),
                                            false, false);
  return fmaxf(__builtin_bit_cast(float, (int)c[0]), __builtin_bit_cast(float, (int)c[1]));
}
__device__ __forceinline__ float quad_sum(float x) {
  auto a = __builtin_amdgcn_permlane16_swap(__builtin_bit_cast(int, x), __builtin_bit_cast(int, x),
                                            false, false);
  x = __builtin_bit_cast(float, (int)a[0]) + __builtin_bit_cast(float, (int)a[1]);
  auto c = __builtin_amdgcn_permlane32_swap(__builtin_bit_cast(int, x), __builtin_bit_cast(int, x),
                                            false, false);
  return __builtin_bit_cast(float, (int)c[0]) + __builtin_bit_cast(float, (int)c[1]);
}

// V tile swizzle: 16-byte chunk cc of row R lives at cc ^ vswz(R), so the 16
// lanes of a quad in a transposing read (rows 4q..4q+3, two chunks each) hit 8
// different bank groups. K tile: cc ^ (R & 7), so the A-fragment reads of rows
// 0..7 (one chunk each) do.
__device__ __forceinline__ int vswz(int R) { return ((R & 3) << 1) | ((R >> 2) & 1); }

__device__ __forceinline__ int wave_incl_scan(int x, int lane) {
#pragma unroll
  for (int off = 1; off < 64; off <<= 1) {
    const int y = __shfl_up(x, off);
    if (lane >= off) x += y;
  }
  return x;
}

// NBUF: ring slots (chunks in flight + 1), (NBUF - 1) * 2 * LPC <= 63 so the
// vector-memory counter can track them all. OCC: waves per SIMD the register
// allocation is held to. POL: cache policy of the K/V loads.
template <typename T, int D, int NBUF, int OCC, int POL>
__global__ void __launch_bounds__(64) __attribute__((amdgpu_waves_per_eu(OCC, OCC)))
partition_stream_kernel(Params p) {
  typedef Mx<T> M;
  typedef typename M::v8 V8;
  typedef typename M::v4 V4;
  typedef Cfg<D> C;
  constexpr int LPC = C::LPC, KS = C::KS, MB = C::MB;
  static_assert((NBUF - 1) * 2 * LPC <= 63, "ring deeper than the vector-memory counter");

  constexpr bool kQLds = D == 256;  // Q' fragments in LDS for d = 256, registers otherwise
  __shared__ __attribute__((aligned(16))) uint16_t s_k[16 * D];
  __shared__ __attribute__((aligned(16))) uint16_t s_v[16 * D];
  __shared__ __attribute__((aligned(16))) V8 s_q[kQLds ? 2 : 1][kQLds ? KS : 1][64];

  const int lane = threadIdx.x;
  const int r = lane & 15, q = lane >> 4;
  const int G = p.G, Hkv = p.Hkv, PART = p.part;
  const int CPP = PART >> 4;  // chunks per partition

  // ---- 1. partitions per sequence and this wave's item range ---------------
  // np(b) = max(1, ceil(L_b / PART)) (an empty sequence still has one item: it
  // writes zeros). Items of sequence b: Hkv * np(b).
  const int nwin = (p.B + 63) >> 6;
  int npw[kMaxWindows];
  int tot = 0;
#pragma unroll
  for (int wi = 0; wi < kMaxWindows; ++wi) {
    int np = 0;
    if (wi < nwin) {
      const int b = wi * 64 + lane;
      if (b < p.B) {
        const int L = clamped_len(p, b, blockIdx.x == 0);
        np = L == 0 ? 1 : (L + PART - 1) / PART;
      }
    }
    npw[wi] = np;
  }
#pragma unroll
  for (int wi = 0; wi < kMaxWindows; ++wi) {
    int s = npw[wi];
#pragma unroll
    for (int off = 32; off >= 1; off >>= 1) s += __shfl_xor(s, off);
    tot += s;  // uniform
  }
  const int64_t n_items = (int64_t)tot * Hkv;
  int64_t i = n_items * blockIdx.x / gridDim.x;
  const int64_t i_end = n_items * (blockIdx.x + 1) / gridDim.x;
  if (i >= i_end) return;

  // sequence holding item i: P(b) <= i / Hkv < P(b + 1)
  int b = 0, Pb = 0, npb = 1;
  {
    const int x = (int)(i / Hkv);
    int carry = 0;
    bool found = false;
#pragma unroll
    for (int wi = 0; wi < kMaxWindows; ++wi) {
      if (!found && wi < nwin) {
        const int incl = wave_incl_scan(npw[wi], lane) + carry;
        const uint64_t hit = __ballot(incl > x && npw[wi] > 0);
        if (hit) {
          const int src = __builtin_ctzll(hit);
          b = wi * 64 + src;
          npb = __shfl(npw[wi], src);
          Pb = __shfl(incl, src) - npb;
          found = true;
        }
        carry = __shfl(incl, 63);
      }
    }
  }
  int L = clamped_len(p, b, false);

  const int bsm = (1 << p.bs_log2) - 1;
  const int rowL = lane / C::CPR;  // row within a load instruction
  const int cc = lane % C::CPR;    // 16-byte chunk of the row this lane loads
  const int tj = r >> 2, tk = r & 3;

  // byte offsets of this lane's 16-byte piece of row s*RPI + rowL in a chunk
  const int kst_bytes = (int)(p.kst * (int)sizeof(T)), vst_bytes = (int)(p.vst * (int)sizeof(T));
  int koffs[LPC], voffs[LPC];
#pragma unroll
  for (int s = 0; s < LPC; ++s) {
    koffs[s] = (s * C::RPI + rowL) * kst_bytes + 16 * cc;
    voffs[s] = (s * C::RPI + rowL) * vst_bytes + 16 * cc;
  }

  // ---- 2. segments: runs of items with the same (b, KV head) ----------------
  while (i < i_end) {
    const int e = (int)(i - (int64_t)Pb * Hkv);
    const int hk = e / npb;
    const int pf = e - hk * npb;
    const int pl = (int)min<int64_t>((int64_t)npb, pf + (i_end - i));

    if (L == 0) {  // empty context: zeros for the group's heads
      for (int k = lane; k < G * D / 4; k += 64) {
        const int g = k / (D / 4), c4 = k % (D / 4);
        *(float4*)(p.out + ((int64_t)b * p.Hq + hk * G + g) * D + 4 * c4) = make_float4(0, 0, 0, 0);
      }
    } else {
      const int T0 = pf * PART;
      const int T1 = min(L, pl * PART);
      const int nch = (T1 - T0 + 15) >> 4;
      const int32_t* trow = p.table + (int64_t)b * p.MBS;
      const char* kbase = (const char*)p.k + (int64_t)hk * p.ksh * (int)sizeof(T);
      const char* vbase = (const char*)p.v + (int64_t)hk * p.vsh * (int)sizeof(T);

      // block id of chunk cw + lane (invalid -> -1, reported)
      auto load_ids = [&](int cw) {
        int id = -1;
        const int c = cw + lane;
        if (c < nch) {
          id = trow[(T0 + 16 * c) >> p.bs_log2];
          if (id < 0 || id >= p.NB) {
            if (p.status) atomicOr(p.status, kStatusBadBlock);
            id = -1;
          }
        }
        return id;
      };
      int cw = 0;
      int idv = load_ids(0);
      int idn = nch > 64 ? load_ids(64) : -1;

      // Q' fragments of head r (zero for padded heads)
      V8 qhi[kQLds ? 1 : KS], qlo[kQLds ? 1 : KS];
      {
        const bool hv = r < G;
        const float* qp = p.q + ((int64_t)b * p.Hq + hk * G + (hv ? r : 0)) * D + 8 * q;
#pragma unroll
        for (int ks = 0; ks < KS; ++ks) {
          const float4 a = hv ? *(const float4*)(qp + 32 * ks) : make_float4(0, 0, 0, 0);
          const float4 c = hv ? *(const float4*)(qp + 32 * ks + 4) : make_float4(0, 0, 0, 0);
          const float x[8] = {a.x, a.y, a.z, a.w, c.x, c.y, c.z, c.w};
          V8 hi, lo;
#pragma unroll
          for (int k = 0; k < 8; ++k) {
            const float y = x[k] * p.qscale;
            const T h = (T)y;
            hi[k] = h;
            lo[k] = (T)(y - (float)h);
          }
          if constexpr (kQLds) {
            s_q[0][ks][lane] = hi;
            s_q[1][ks][lane] = lo;
          } else {
            qhi[ks] = hi;
            qlo[ks] = lo;
          }
        }
      }

      // issue the loads of chunk cn into one ring slot; returns the chunk's
      // number of attended rows (0 behind an invalid table entry). The buffer
      // descriptors cover exactly those rows: lanes whose row lies beyond them
      // read zeros without a memory access.
      auto issue = [&](int cn, uint4 (&rk)[LPC], uint4 (&rv)[LPC]) -> int {
        if (cn >= cw + 64) {  // the issue pointer enters the next window of ids
          cw += 64;
          idv = idn;
          idn = cw + 64 < nch ? load_ids(cw + 64) : -1;
        }
        const int id = __builtin_amdgcn_readlane(idv, cn - cw);
        const int tok0 = T0 + 16 * cn;
        const int rows = id >= 0 ? min(16, T1 - tok0) : 0;
        const int64_t row0 = id >= 0 ? (int64_t)(tok0 & bsm) : 0;
        const int64_t idc = id >= 0 ? (int64_t)id : 0;
        const __amdgpu_buffer_rsrc_t rsk = uniform_rsrc(
            kbase + (idc * p.ksb + row0 * p.kst) * (int)sizeof(T), rows * kst_bytes);
        const __amdgpu_buffer_rsrc_t rsv = uniform_rsrc(
            vbase + (idc * p.vsb + row0 * p.vst) * (int)sizeof(T), rows * vst_bytes);
#pragma unroll
        for (int s = 0; s < LPC; ++s) {
          rk[s] = buf_load<POL>(rsk, koffs[s]);
          rv[s] = buf_load<POL>(rsv, voffs[s]);
        }
        return rows;
      };

      f32x4 acc[MB];
#pragma unroll
      for (int k = 0; k < MB; ++k) acc[k] = f32x4{0.f, 0.f, 0.f, 0.f};
      float m = -INFINITY, l = 0.f;

      // write the finished partition pp's state and reset
      auto flush = [&](int pp) {
        const float lt = quad_sum(l);
        if (r < G) {
          const int h = hk * G + r;
          if (npb == 1) {
            const float inv = lt > 0.f ? 1.f / lt : 0.f;
            float* op = p.out + ((int64_t)b * p.Hq + h) * D + 4 * q;
#pragma unroll
            for (int mb = 0; mb < MB; ++mb) {
              const f32x4 o = acc[mb] * inv;
              *(float4*)(op + 16 * mb) = make_float4(o[0], o[1], o[2], o[3]);
            }
          } else {
            const int64_t row = ((int64_t)b * p.Hq + h) * p.pmax + pp;
            float* ap = p.ws_acc + row * D + 4 * q;
#pragma unroll
            for (int mb = 0; mb < MB; ++mb)
              *(float4*)(ap + 16 * mb) = make_float4(acc[mb][0], acc[mb][1], acc[mb][2], acc[mb][3]);
            if (q == 0) {
              p.ws_m[row] = m;
              p.ws_l[row] = lt;
            }
          }
        }
#pragma unroll
        for (int k = 0; k < MB; ++k) acc[k] = f32x4{0.f, 0.f, 0.f, 0.f};
        m = -INFINITY;
        l = 0.f;
      };

      // fold one chunk (its rows in a ring slot, `rows` of them attended)
      auto consume = [&](int rows, const uint4 (&rk)[LPC], const uint4 (&rv)[LPC]) {
        // stage K and V rows in LDS
#pragma unroll
        for (int s = 0; s < LPC; ++s) {
          const int R = s * C::RPI + rowL;
          *(uint4*)(s_k + R * D + 8 * (cc ^ (R & 7))) = rk[s];
          *(uint4*)(s_v + R * D + 8 * (cc ^ vswz(R))) = rv[s];
        }
        // scores of the 16 tokens: lane (q, r) gets tokens 4q..4q+3 of head r
        f32x4 st = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int ks = 0; ks < KS; ++ks) {
          const V8 a = *(const V8*)(s_k + r * D + 8 * ((4 * ks + q) ^ (r & 7)));
          if constexpr (kQLds) {
            st = M::mma32(a, s_q[0][ks][lane], st);
            st = M::mma32(a, s_q[1][ks][lane], st);
          } else {
            st = M::mma32(a, qhi[ks], st);
            st = M::mma32(a, qlo[ks], st);
          }
        }
        float sv[4];
#pragma unroll
        for (int k = 0; k < 4; ++k) sv[k] = (4 * q + k < rows) ? st[k] : -INFINITY;

        // running softmax state of head r (same in all four quads); the
        // reference max m is raised only when a score passes m + 8
        const float mt = quad_max(fmaxf(fmaxf(sv[0], sv[1]), fmaxf(sv[2], sv[3])));
        const bool raise = mt > m + 8.f;
        if (__ballot(raise)) {
          const float mn = raise ? mt : m;
          const float alpha = exp2_fast(m - (mn == -INFINITY ? 0.f : mn));
          l *= alpha;
#pragma unroll
          for (int k = 0; k < MB; ++k) acc[k] *= alpha;
          m = mn;
        }
        const float mu = m == -INFINITY ? 0.f : m;
        float pv[4];
#pragma unroll
        for (int k = 0; k < 4; ++k) pv[k] = exp2_fast(sv[k] - mu);
        l += (pv[0] + pv[1]) + (pv[2] + pv[3]);

        // P^T fragment (k-slot j = token 4q + j) as hi + lo
        typename M::e4 ph, pl2;
#pragma unroll
        for (int k = 0; k < 4; ++k) {
          const T h = (T)pv[k];
          ph[k] = h;
          pl2[k] = (T)(pv[k] - (float)h);
        }
        const V4 phi = M::pack(ph), plo = M::pack(pl2);

        // O^T += V^T P^T; lane (q, 4j + k) points the transposing read at row
        // 4q + j, columns 16 mb + 4k .. +3 of the V tile
#pragma unroll
        for (int mb = 0; mb < MB; ++mb) {
          const int pc = 2 * (mb ^ tj) + ((tk >> 1) ^ (q & 1));
          const s16x4 a4 = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
              (lds_s16x4*)(s_v + (4 * q + tj) * D + 8 * pc + 4 * (tk & 1)));
          const V4 av = __builtin_bit_cast(V4, a4);
          acc[mb] = M::mma16(av, phi, acc[mb]);
          acc[mb] = M::mma16(av, plo, acc[mb]);
        }
      };

      // ---- the ring: slot c % NBUF holds chunk c; chunk c + NBUF - 1 is issued
      // just before chunk c is consumed
      uint4 rk[NBUF][LPC], rv[NBUF][LPC];
      int rows[NBUF];
      static_for<0, NBUF - 1>([&](auto S) {
        constexpr int s = decltype(S)::value;
        rows[s] = s < nch ? issue(s, rk[s], rv[s]) : 0;
      });
      for (int cb = 0; cb < nch; cb += NBUF) {
        static_for<0, NBUF>([&](auto S) {
          constexpr int s = decltype(S)::value;
          constexpr int sn = (s + NBUF - 1) % NBUF;
          const int c = cb + s;
          if (c < nch) {
            if (c + NBUF - 1 < nch) rows[sn] = issue(c + NBUF - 1, rk[sn], rv[sn]);
            consume(rows[s], rk[s], rv[s]);
            if ((c + 1) % CPP == 0 || c + 1 == nch) flush(pf + c / CPP);
          }
        });
      }
    }

    // advance to the next segment
    i += pl - pf;
    if (pl == npb && hk + 1 == Hkv && i < i_end) {
      Pb += npb;
      ++b;
      L = clamped_len(p, b, false);
      npb = L == 0 ? 1 : (L + PART - 1) / PART;
    }
  }
}

template <typename T, int D, int NBUF, int OCC, int POL>
hipError_t launch_t(const Params& p, int cus, hipStream_t s) {
  const int64_t items = (int64_t)p.B * p.Hkv * p.pmax;
  const int64_t slots = 4LL * OCC * cus;  // one wave per SIMD slot
  const int waves = (int)(items < slots ? items : slots);
  hipLaunchKernelGGL((partition_stream_kernel<T, D, NBUF, OCC, POL>), dim3(waves), dim3(64), 0, s,
                     p);
  return hipGetLastError();
}

// Ring depth / occupancy variants per head_dim (variant 0 is the default).
template <typename T, int POL>
hipError_t launch_v(const Params& p, int cus, int variant, hipStream_t s) {
  switch (p.D) {
    case 64:
      if (variant == 1) return launch_t<T, 64, 12, 1, POL>(p, cus, s);
      if (variant == 2) return launch_t<T, 64, 4, 4, POL>(p, cus, s);
      return launch_t<T, 64, 6, 2, POL>(p, cus, s);
    case 128:
      if (variant == 1) return launch_t<T, 128, 6, 1, POL>(p, cus, s);
      if (variant == 2) return launch_t<T, 128, 2, 3, POL>(p, cus, s);
      return launch_t<T, 128, 3, 2, POL>(p, cus, s);
    case 256:
      if (variant == 1) return launch_t<T, 256, 2, 1, POL>(p, cus, s);
      if (variant == 2) return launch_t<T, 256, 4, 1, POL>(p, cus, s);
      return launch_t<T, 256, 3, 1, POL>(p, cus, s);
  }
  return hipErrorInvalidValue;
}

template <typename T>
hipError_t launch_d(const Params& p, int cus, int variant, bool nt, hipStream_t s) {
  return nt ? launch_v<T, 2>(p, cus, variant, s) : launch_v<T, 0>(p, cus, variant, s);
}

}  // namespace

bool stream_supports(int dtype, int D, int G, int block_size, int batch) {
  return mfma_supports(dtype, D, G) && block_size >= 16 && batch <= kMaxWindows * 64;
}

hipError_t launch_partition_stream(const Params& p, int dtype, int cus, int variant, bool nt,
                                   hipStream_t s) {
  if (dtype == 1) return launch_d<_Float16>(p, cus, variant, nt, s);
  if (dtype == 2) return launch_d<__bf16>(p, cus, variant, nt, s);
  return hipErrorInvalidValue;
}

}  // namespace pa
