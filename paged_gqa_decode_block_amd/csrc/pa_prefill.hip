// pa_prefill.hip -- paged varlen prefill on the matrix cores (gfx950).
//
// Sequence b has q_len_b query rows, rows cu_q[b] .. cu_q[b+1]-1 of the packed
// q ([total_q, H_q, d], the varlen indexing of the paged-attention docs page),
// and L_b keys in the paged pool (the new tokens already written there). With
// the causal rule, its query i sits at position L_b - q_len_b + i and attends
// tokens [0, L_b - q_len_b + i]; a query with no token to attend gets zeros.
// Otherwise every query attends all L_b tokens.
//
// One workgroup per eight (16-row query tile, query head) units of one KV
// head: 8 / hh consecutive tiles of a sequence times hh of the KV head's query
// heads (hh = 8, or the largest power of two dividing G, so that no unit is
// empty). Its threads load each 16-token chunk of K and V once (16-byte
// pieces, raw buffer loads through descriptors cut to the chunk's attended
// rows, an invalid table entry never dereferenced) into a ring of chunks in
// registers, and stage two consecutive chunks into one of two 32-token LDS
// tiles; after one barrier per tile every wave folds its units against it:
//
//   scores  S^T[token, row] = K[token, :] . Q'[row, :]       16x16x32 MFMAs,
//           two 16-token halves
//   update  running max m, sum l, output per row and head (base 2, lazily
//           rescaled)
//   output  O^T[dim, row] += V^T[dim, token] . P^T[token, row]  16x16x32 over
//           the 32 tokens
//
// with a tile's 16 rows as the MFMA columns and Q' and P in hi + lo 16-bit
// parts. (On gfx950 a 16x16x16 bf16 MFMA takes as long as a 16x16x32 one, so
// the output product runs on 32-token tiles.) The workgroup walks the tokens
// up to its last tile's last row's key end; a token is masked per column, so
// each row ends at its own causal bound. No partial state leaves the
// workgroup: each unit is normalised and written at the end.
//
// Requires 16-bit K/V and block_size >= 16.
#include "pa_mfma_util.h"

namespace pa {
namespace {

constexpr int kHeadsPerGroup = 8;  // (tile, head) units per workgroup: 8 / NW per wave

// NW waves per workgroup (4: two heads per wave; 8: one head per wave, half
// the registers, so that d = 256 runs two waves per SIMD), NBUF ring slots,
// OCC waves per SIMD.
template <typename T, int D, int NW, int NBUF, int OCC, int QO>
__global__ void __launch_bounds__(64 * NW) __attribute__((amdgpu_waves_per_eu(OCC, OCC)))
prefill_kernel(Params p, const int32_t* __restrict__ cu_q, int causal, int nhg, int hh,
               int ntiles) {
  typedef Mx<T> M;
  typedef typename M::v8 V8;
  typedef typename M::v4 V4;
  constexpr int KS = D / 32, MB = D / 16;
  constexpr int kThreads = 64 * NW;
  constexpr int PPT = 4 * D / kThreads;  // 16-byte pieces of a chunk per thread (4 D of them)
  constexpr int HPW = kHeadsPerGroup / NW;
  static_assert(PPT * kThreads == 4 * D, "the workgroup loads a chunk in whole pieces");
  static_assert((NBUF - 1) * PPT <= 60, "ring deeper than the vector-memory counter");
  // 32-row K and V tiles with the decode's padded rows (one 32-byte pad per
  // 256-byte bank line: conflict-free fragment reads and staging writes)
  typedef TileRows<D> TR;
  constexpr int kTile = 32 * D + (32 / TR::RPL) * TR::PAD;
  constexpr int kHalf = 16 * D + (16 / TR::RPL) * TR::PAD;  // TR::row(16 + x) - TR::row(x)
  __shared__ __attribute__((aligned(16))) uint16_t s_k[2][kTile];
  __shared__ __attribute__((aligned(16))) uint16_t s_v[2][kTile];

  const int tid = threadIdx.x;
  const int w = tid >> 6, lane = tid & 63;
  const int r = lane & 15, q = lane >> 4;
  // The workgroup's 8 (tile, head) units: tpw = 8 / hh consecutive 16-row
  // tiles times hh query heads of KV head hk (heads g0 .. g0 + hh - 1 of its
  // group). Each K/V chunk it loads serves all eight.
  const int tpw = kHeadsPerGroup / hh;
  const int b = blockIdx.z;
  const int hk = (int)blockIdx.y / nhg, g0 = ((int)blockIdx.y % nhg) * hh;
  const int hcount = min(hh, p.G - g0);
  const int pw0 = 16 * tpw * (int)blockIdx.x;  // first row of the workgroup's tiles
  const int r0 = cu_q[b];
  const int ql = cu_q[b + 1] - r0;
  // rows beyond the grid would be left unwritten: report
  if (blockIdx.x == 0 && blockIdx.y == 0 && tid == 0 && p.status && (ql < 0 || ql > 16 * ntiles))
    atomicOr(p.status, kStatusBadSeqlen);
  if (pw0 >= ql) return;  // the whole workgroup
  const int L = clamped_len(p, b, blockIdx.x == 0 && blockIdx.y == 0 && tid == 0);
  const int plast = min(pw0 + 16 * tpw - 1, ql - 1);
  const int kend = causal ? min(L, max(0, L - ql + plast + 1)) : L;  // the last tile's
  const int nch = (kend + 15) >> 4;

  // slot j of this wave: unit u = w + NW j, tile u / hh, head u % hh. Column r
  // is query position p0s + r of the sequence; its keys are [0, kend_r).
  bool hon[HPW], col_ok[HPW];
  int kend_r[HPW], p0s[HPW], hls[HPW];
  // kfull[j]: the least key end over slot j's valid columns (the whole wave
  // agrees); a 32-token tile ending at or below it needs no mask
  int kfull[HPW];
  V8 qhi[HPW][KS], qlo[HPW][KS];
#pragma unroll
  for (int j = 0; j < HPW; ++j) {
    const int u = w + NW * j, tl = u / hh;
    hls[j] = u - tl * hh;
    p0s[j] = pw0 + 16 * tl;
    col_ok[j] = p0s[j] + r < ql;
    hon[j] = hls[j] < hcount && p0s[j] < ql;
    kend_r[j] = !col_ok[j] ? 0 : causal ? min(L, max(0, L - ql + p0s[j] + r + 1)) : L;
    int kf = col_ok[j] ? kend_r[j] : 0x7fffffff;
#pragma unroll
    for (int off = 1; off < 64; off <<= 1) kf = min(kf, __shfl_xor(kf, off));
    kfull[j] = __builtin_amdgcn_readfirstlane(kf);
    const int h = hk * p.G + g0 + (hon[j] ? hls[j] : 0);
    const int64_t qrow = ((int64_t)(r0 + (col_ok[j] ? p0s[j] + r : 0)) * p.Hq + h) * D + 8 * q;
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) {
      const float4 a = load_q4<QO>(p, qrow + 32 * ks);
      const float4 c = load_q4<QO>(p, qrow + 32 * ks + 4);
      const float x[8] = {a.x, a.y, a.z, a.w, c.x, c.y, c.z, c.w};
#pragma unroll
      for (int k = 0; k < 8; ++k) {
        const float y = col_ok[j] ? x[k] * p.qscale : 0.f;
        const T hh = (T)y;
        qhi[j][ks][k] = hh;
        qlo[j][ks][k] = (T)(y - (float)hh);
      }
    }
  }

  // the pieces this thread loads: piece i = tid + 64 NW k of the chunk's 4 D
  // (K pieces first): row, 16-byte column and whether it is V
  const int bsm = (1 << p.bs_log2) - 1;
  const int kst_bytes = (int)(p.kst * (int)sizeof(T)), vst_bytes = (int)(p.vst * (int)sizeof(T));
  int poff[PPT], plds[PPT];
  bool pisv[PPT];
#pragma unroll
  for (int k = 0; k < PPT; ++k) {
    const int i = tid + kThreads * k;
    // a wave's 64 pieces are consecutive and 2 D is a multiple of 64, so K or V
    // is the same across the wave: made visibly uniform for the descriptor choice
    pisv[k] = __builtin_amdgcn_readfirstlane(i >= 2 * D ? 1 : 0) != 0;
    const int jj = pisv[k] ? i - 2 * D : i;
    const int row = jj / (D / 8), cc = jj % (D / 8);
    poff[k] = row * (pisv[k] ? vst_bytes : kst_bytes) + 16 * cc;
    plds[k] = TR::row(row) + 8 * cc;
  }

  const int32_t* trow = p.table + (int64_t)b * p.MBS;
  const char* kbase = (const char*)p.k + (int64_t)hk * p.ksh * (int)sizeof(T);
  const char* vbase = (const char*)p.v + (int64_t)hk * p.vsh * (int)sizeof(T);
  const int nblk = (kend + bsm) >> p.bs_log2;
  const __amdgpu_buffer_rsrc_t rst = uniform_rsrc((const char*)trow, nblk * 4);
  auto fetch_id = [&](int cn) -> int {
    return (int)__builtin_amdgcn_raw_buffer_load_b32(rst, ((16 * cn) >> p.bs_log2) * 4, 0, 0);
  };
  int idr[NBUF];
  static_for<0, NBUF>([&](auto S) { idr[decltype(S)::value] = fetch_id(decltype(S)::value); });

  int bad_block = 0;
  // (the lambdas are forced inline: called out of line, their ring arguments
  // would live in scratch memory)
  auto issue = [&](int cn, uint4 (&pc)[PPT], int& ids) __attribute__((always_inline)) {
    int id = __builtin_amdgcn_readfirstlane(ids);
    if (cn >= nch) {
      id = -1;
    } else if (id < 0 || id >= p.NB) {
      bad_block = 1;
      id = -1;
    }
    const int tok0 = 16 * cn;
    const int rows = id >= 0 ? min(16, kend - tok0) : 0;
    const int64_t row0 = id >= 0 ? (int64_t)(tok0 & bsm) : 0;
    const int64_t idc = id >= 0 ? (int64_t)id : 0;
    const __amdgpu_buffer_rsrc_t rsk =
        uniform_rsrc(kbase + (idc * p.ksb + row0 * p.kst) * (int)sizeof(T), rows * kst_bytes);
    const __amdgpu_buffer_rsrc_t rsv =
        uniform_rsrc(vbase + (idc * p.vsb + row0 * p.vst) * (int)sizeof(T), rows * vst_bytes);
#pragma unroll
    for (int k = 0; k < PPT; ++k) {
      pc[k] = buf_load<2>(pisv[k] ? rsv : rsk, poff[k]);  // a scalar select
    }
    ids = fetch_id(cn + NBUF);
  };

  f32x4 acc[HPW][MB];
  float m[HPW], l[HPW];
#pragma unroll
  for (int j = 0; j < HPW; ++j) {
#pragma unroll
    for (int k = 0; k < MB; ++k) acc[j][k] = f32x4{0.f, 0.f, 0.f, 0.f};
    m[j] = -INFINITY;
    l[j] = 0.f;
  }
  const int tj = r >> 2, tk = r & 3;

  // fold 32-token tile tc (tokens 32 tc .., staged in LDS tile `buf`) into
  // head slot j. P^T k-slot i of lane (q, r) holds token 16 (i / 4) + 4 q + i % 4,
  // the score MFMA's output layout of the two halves.
  auto consume = [&](int tc, int buf, int j) __attribute__((always_inline)) {
    const uint16_t* sk = s_k[buf];
    const uint16_t* sv_ = s_v[buf];
    f32x4 st[2] = {f32x4{0.f, 0.f, 0.f, 0.f}, f32x4{0.f, 0.f, 0.f, 0.f}};
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) {
#pragma unroll
      for (int tau = 0; tau < 2; ++tau) {
        const V8 a = *(const V8*)(sk + tau * kHalf + TR::row(r) + 8 * (4 * ks + q));
        st[tau] = M::mma32(a, qhi[j][ks], st[tau]);
        st[tau] = M::mma32(a, qlo[j][ks], st[tau]);
      }
    }
    float sv[8];
    if (32 * tc + 32 <= kfull[j]) {  // every valid column attends the whole tile
#pragma unroll
      for (int i = 0; i < 8; ++i) sv[i] = st[i >> 2][i & 3];
    } else {
#pragma unroll
      for (int i = 0; i < 8; ++i)
        sv[i] = (32 * tc + 16 * (i >> 2) + 4 * q + (i & 3) < kend_r[j]) ? st[i >> 2][i & 3] : -INFINITY;
    }
    float mx = sv[0];
#pragma unroll
    for (int i = 1; i < 8; ++i) mx = fmaxf(mx, sv[i]);
    const float mt = quad_max(mx);
    const bool raise = mt > m[j] + 8.f;
    if (__ballot(raise)) {
      const float mn = raise ? mt : m[j];
      const float alpha = exp2_fast(m[j] - (mn == -INFINITY ? 0.f : mn));
      l[j] *= alpha;
#pragma unroll
      for (int k = 0; k < MB; ++k) acc[j][k] *= alpha;
      m[j] = mn;
    }
    const float mu = m[j] == -INFINITY ? 0.f : m[j];
    float pv[8];
#pragma unroll
    for (int i = 0; i < 8; ++i) pv[i] = exp2_fast(sv[i] - mu);
    l[j] += ((pv[0] + pv[1]) + (pv[2] + pv[3])) + ((pv[4] + pv[5]) + (pv[6] + pv[7]));
    V8 phi, plo;
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      const T hh = (T)pv[i];
      phi[i] = hh;
      plo[i] = (T)(pv[i] - (float)hh);
    }
    const int vbase = TR::row(4 * q + tj) + 8 * (tk >> 1) + 4 * (tk & 1);
#pragma unroll
    for (int mb = 0; mb < MB; ++mb) {
      const int o = vbase + 16 * mb;
      const s16x4 lo4 = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4*)(sv_ + o));
      const s16x4 hi4 = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4*)(sv_ + kHalf + o));
      const V8 av = __builtin_bit_cast(V8, __builtin_shufflevector(lo4, hi4, 0, 1, 2, 3, 4, 5, 6, 7));
      acc[j][mb] = M::mma32(av, phi, acc[j][mb]);
      acc[j][mb] = M::mma32(av, plo, acc[j][mb]);
    }
  };

  // the ring: chunk c + NBUF - 1 is issued just before chunk c is staged
  // (unconditionally: past the end the descriptors are empty, so an odd last
  // chunk is paired with zeros). Chunk c goes to half c % 2 of 32-token LDS
  // tile (c / 2) % 2; the barrier after a tile's second half also means every
  // wave is done with the tile before, so the other tile is free.
  const int nch2 = (nch + 1) & ~1;
  uint4 ring[NBUF][PPT];
  static_for<0, NBUF - 1>([&](auto S) {
    constexpr int s = decltype(S)::value;
    issue(s, ring[s], idr[s]);
  });
  for (int cb = 0; cb < nch2; cb += NBUF) {
    static_for<0, NBUF>([&](auto S) {
      constexpr int s = decltype(S)::value;
      constexpr int sn = (s + NBUF - 1) % NBUF;
      const int c = cb + s;
      issue(c + NBUF - 1, ring[sn], idr[sn]);
      __builtin_amdgcn_sched_barrier(0);
      if (c < nch2) {
        const int buf = (c >> 1) & 1, half = (c & 1) * kHalf;
#pragma unroll
        for (int k = 0; k < PPT; ++k) {
          uint16_t* dst = pisv[k] ? s_v[buf] : s_k[buf];
          *(uint4*)(dst + half + plds[k]) = ring[s][k];
        }
        if (c & 1) {
          __syncthreads();
#pragma unroll
          for (int j = 0; j < HPW; ++j)
            if (hon[j]) consume(c >> 1, buf, j);
        }
      }
    });
  }

#pragma unroll
  for (int j = 0; j < HPW; ++j) {
    const float lt = quad_sum(l[j]);
    if (hon[j] && col_ok[j]) {
      const float inv = lt > 0.f ? 1.f / lt : 0.f;
      const int h = hk * p.G + g0 + hls[j];
      const int64_t orow = ((int64_t)(r0 + p0s[j] + r) * p.Hq + h) * D + 4 * q;
#pragma unroll
      for (int mb = 0; mb < MB; ++mb) {
        const f32x4 o = acc[j][mb] * inv;
        store_out4<QO>(p, orow + 16 * mb, o[0], o[1], o[2], o[3]);
      }
    }
  }
  if (bad_block && tid == 0 && p.status) atomicOr(p.status, kStatusBadBlock);
}

// {waves per workgroup, ring slots, waves per SIMD} per head_dim
constexpr int kPrefillCfg[3][3] = {{4, 6, 2}, {8, 4, 4}, {8, 4, 2}};
constexpr int pdim(int D) { return D == 64 ? 0 : D == 128 ? 1 : 2; }

template <typename T, int D, int QO>
hipError_t launch_p(const Params& p, const int32_t* cu_q, int max_q, int causal, hipStream_t s) {
  constexpr int NW = kPrefillCfg[pdim(D)][0], NB_ = kPrefillCfg[pdim(D)][1],
                OCC = kPrefillCfg[pdim(D)][2];
  // heads per workgroup: 8 when they divide G; else the largest power of two
  // dividing G, with 8 / hh tiles per workgroup so that no unit is idle, if
  // there are that many tiles (else 8, the last group partly empty)
  const int ntiles = (max_q + 15) / 16;
  int hh = kHeadsPerGroup;
  if (p.G % kHeadsPerGroup) {
    int h2 = 1;
    while (2 * h2 < kHeadsPerGroup && p.G % (2 * h2) == 0) h2 *= 2;
    if (ntiles >= kHeadsPerGroup / h2) hh = h2;
  }
  const int tpw = kHeadsPerGroup / hh;
  const int nhg = (p.G + hh - 1) / hh;
  dim3 grid((ntiles + tpw - 1) / tpw, p.Hkv * nhg, p.B);
  hipLaunchKernelGGL((prefill_kernel<T, D, NW, NB_, OCC, QO>), grid, dim3(64 * NW), 0, s, p,
                     cu_q, causal, nhg, hh, ntiles);
  return hipGetLastError();
}

template <typename T>
hipError_t launch_pd(const Params& p, const int32_t* cu_q, int max_q, int causal, hipStream_t s) {
  const bool bf = p.qo_bf16 != 0;
  switch (p.D) {
    case 64: return bf ? launch_p<T, 64, 1>(p, cu_q, max_q, causal, s)
                       : launch_p<T, 64, 0>(p, cu_q, max_q, causal, s);
    case 128: return bf ? launch_p<T, 128, 1>(p, cu_q, max_q, causal, s)
                        : launch_p<T, 128, 0>(p, cu_q, max_q, causal, s);
    case 256: return bf ? launch_p<T, 256, 1>(p, cu_q, max_q, causal, s)
                        : launch_p<T, 256, 0>(p, cu_q, max_q, causal, s);
  }
  return hipErrorInvalidValue;
}

}  // namespace

hipError_t launch_prefill(const Params& p, int dtype, const int32_t* cu_q, int max_q, int causal,
                          hipStream_t s) {
  if (max_q <= 0 || p.B <= 0) return hipSuccess;
  if (dtype == 1) return launch_pd<_Float16>(p, cu_q, max_q, causal, s);
  if (dtype == 2) return launch_pd<__bf16>(p, cu_q, max_q, causal, s);
  return hipErrorInvalidValue;
}

}  // namespace pa
