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
// empty). All the workgroups of one (sequence, KV head) read the same K and V,
// so they are placed on one XCD, whose L2 serves the repeats (the loads keep
// the default cache policy); an XCD with 4 to 64 pairs takes them longest
// first, so that its last workgroups are short. Its threads load each
// 16-token chunk of K and V once (16-byte pieces, raw buffer loads through
// descriptors cut to the chunk's attended rows, an invalid table entry never
// dereferenced) into a ring of chunks in registers, and stage consecutive
// chunks into one of two LDS tiles of 32 tokens (64 for bf16 q at d = 256);
// after one barrier per tile every wave folds its units against each 32-token
// half of it:
//
//   scores  S^T[token, row] = K[token, :] . Q'[row, :]       16x16x32 MFMAs,
//           two 16-token halves
//   update  running max m, sum l, output per row and head (base 2, lazily
//           rescaled)
//   output  O^T[dim, row] += V^T[dim, token] . P^T[token, row]  16x16x32 over
//           the 32 tokens
//
// with a tile's 16 rows as the MFMA columns. (On gfx950 a 16x16x16 bf16 MFMA
// takes as long as a 16x16x32 one, so the output product runs on 32-token
// tiles.)
//
// Operand precision. Q': bf16 q over bf16 K is exact in bf16 (sign(scale) q),
// so the scores are exact fp32 sums and |scale| log2 e is applied to them;
// otherwise Q' = q scale log2 e goes in hi + lo 16-bit parts (~16 significant
// bits, two MFMAs). P: the probabilities (at most 2^8 with the lazy max) go to
// fp16, 11 significant bits, and the row sums add the rounded values, so the
// output is a convex combination of V rows whose weights carry a relative
// error of at most 2^-11: within the fp16/bf16 tolerance even for a sharply
// peaked softmax. bf16 V is converted to fp16 as it is staged, without a
// range check: a bf16 value of magnitude 2^16 or more (beyond fp16's finite
// range) becomes an infinity there, and any product with it (0 x inf
// included) leaves a non-finite output. A workgroup that finds a non-finite
// value among its outputs folds all its tiles again with V staged as bf16 and
// P in bf16 hi + lo parts (~16 significant bits); non-finite inputs lead
// there too and give the same result on that pass. The workgroup walks the
// tokens up to its last tile's last row's key end; a token is masked per
// column, so each row ends at its own causal bound. No partial state leaves
// the workgroup: each unit is normalised and written at the end.
//
// Key split. When the work items (eight units each) would fill the compute
// units one and a half times or less on a round (the last round at most half
// full), the items of that last round are split in two halves of their key
// tiles, so the GPU runs the whole items and then the halves instead of a
// second full round. Both halves store their state (max, sum and unnormalised
// output per unit, as the folds left them) in the workspace and count in on
// the item's arrival counter; the second to arrive merges the two states with
// the max-rescaling combine (page "Paged Attention Kernel Architecture for
// BI-V100", section 2), resets the counter and writes the output.
//
// Requires 16-bit K/V and block_size >= 16.
#include "pa_mfma_util.h"

namespace pa {
namespace {

constexpr int kHeadsPerGroup = 8;  // (tile, head) units per workgroup: 8 / NW per wave
constexpr int kXcds = 8;            // gfx950 (MI350 series): eight XCDs, each with its own L2

// Device-scope cache bits (SC1 set, SC0 clear on gfx950) of the key split's
// state traffic: a store completes only at the device-coherent level, a load
// is served from there (not from a line another XCD's write left stale in this
// XCD's L2).
constexpr int kScDevice = 16;

// Eight bf16 values (16 bytes) as fp16, exact where fp16 has the value (below
// 2^-14 it keeps fp16's subnormal grid; from 2^16 on, infinite).
__device__ __forceinline__ uint4 bf16x8_to_f16(uint4 w) {
  typedef _Float16 h2 __attribute__((ext_vector_type(2)));
  const uint32_t in[4] = {w.x, w.y, w.z, w.w};
  uint32_t out[4];
  float f[8];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    f[2 * i] = __builtin_bit_cast(float, in[i] << 16);
    f[2 * i + 1] = __builtin_bit_cast(float, in[i] & 0xffff0000u);
    out[i] = __builtin_bit_cast(uint32_t, h2{(_Float16)f[2 * i], (_Float16)f[2 * i + 1]});
  }
  return make_uint4(out[0], out[1], out[2], out[3]);
}

// NW waves per workgroup (4: two units per wave, each K and V^T fragment read
// once for both; 8: one unit per wave, half the registers, so that d = 256
// runs two waves per SIMD), NBUF ring slots, OCC waves per SIMD.
//
// Work items per XCD: the first nwhole whole, the next nsplit split in two
// halves (all first halves dispatched, then all second halves); ws_cnt
// [kXcds * nsplit] arrival counters, ws_st the halves' states.
template <typename T, int D, int NW, int NBUF, int OCC, int QO>
__global__ void __launch_bounds__(64 * NW) __attribute__((amdgpu_waves_per_eu(OCC, OCC)))
prefill_kernel(Params p, const int32_t* __restrict__ cu_q, int causal, int nhg, int hh,
               int ntiles, int per, int nwhole, int nsplit, int32_t* __restrict__ ws_cnt,
               float* __restrict__ ws_st) {
  typedef Mx<T> M;
  typedef typename M::v8 V8;
  typedef Mx<_Float16> H;
  typedef typename H::v8 H8;
  typedef _Float16 h2 __attribute__((ext_vector_type(2)));
  constexpr bool kBf = std::is_same<T, __bf16>::value;
  constexpr bool kQ1 = kBf && QO == 1;  // Q' exact in one bf16 part
  constexpr int KS = D / 32, MB = D / 16;
  constexpr int kThreads = 64 * NW;
  constexpr int PPT = 4 * D / kThreads;  // 16-byte pieces of a chunk per thread (4 D of them)
  constexpr int HPW = kHeadsPerGroup / NW;
  static_assert(PPT * kThreads == 4 * D, "the workgroup loads a chunk in whole pieces");
  static_assert((NBUF - 1) * PPT <= 60, "ring deeper than the vector-memory counter");
  // 16 CPT-row K and V tiles with the decode's padded rows (one 32-byte pad
  // per 256-byte bank line: conflict-free fragment reads and staging writes)
  typedef TileRows<D> TR;
  // 16-token chunks per LDS tile: 64-token tiles (one barrier per four
  // chunks) for bf16 q at d = 256, where a workgroup has the compute unit's
  // LDS to itself (measured 1-2 % faster there, slower with fp32 q)
  constexpr int CPT = (D == 256 && QO == 1) ? 4 : 2;
  constexpr int kTile = 16 * CPT * D + (16 * CPT / TR::RPL) * TR::PAD;
  constexpr int kHalf = 16 * D + (16 / TR::RPL) * TR::PAD;  // TR::row(16 + x) - TR::row(x)
  // V tiles hold fp16 (bf16 V converted while staged), or bf16 on the second
  // pass of a workgroup whose first pass left a non-finite output (s_redo)
  __shared__ __attribute__((aligned(16))) uint16_t s_k[2][kTile];
  __shared__ __attribute__((aligned(16))) uint16_t s_v[2][kTile];
  __shared__ int s_redo;
  __shared__ int s_arrived;  // the key split: halves of the item that arrived before this one

  const int tid = threadIdx.x;
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6), lane = tid & 63;  // w: the wave's
  const int r = lane & 15, q = lane >> 4;
  // The workgroup's 8 (tile, head) units: tpw = 8 / hh consecutive 16-row
  // tiles times hh query heads of KV head hk (heads g0 .. g0 + hh - 1 of its
  // group). Each K/V chunk it loads serves all eight.
  const int tpw = kHeadsPerGroup / hh;
  // The per work items of one (sequence, KV head) read the same K and V: they
  // all go to one XCD (workgroup i runs on XCD i mod kXcds), whose L2 then
  // serves the repeated reads. XCD x takes the pairs x, x + kXcds, ...
  // The XCD's work item i (item i % per of the pair at position i / per of
  // its list), whole, or half sp of its key tiles.
  const int xcd = (int)blockIdx.x % kXcds, slot = (int)blockIdx.x / kXcds;
  int wi = slot, sp = -1;
  if (slot >= nwhole) {
    const int h = slot - nwhole;
    wi = nwhole + h % nsplit;
    sp = h / nsplit;
  }
  // With 4 to 64 pairs per XCD the list is taken longest first (by key count,
  // ties in pair order), so that the last workgroups to start are short ones;
  // every wave ranks the pairs itself (one length per lane).
  int pos = wi / per;
  {
    const int npl = (nwhole + nsplit) / per;
    if (npl >= 4 && npl <= 64) {
      const int ln = tid & 63, pr = xcd + kXcds * ln;
      int Lr = -1;  // padding pairs last
      if (ln < npl && pr < p.B * p.Hkv) {
        const int lmax = p.MBS << p.bs_log2;
        Lr = min(max(p.seqlens[pr / p.Hkv], 0), lmax);
      }
      int rank = 0;
      for (int j = 0; j < npl; ++j) {
        const int Lj = __shfl(Lr, j);
        rank += (Lj > Lr || (Lj == Lr && j < ln)) ? 1 : 0;
      }
      const uint64_t hit = __ballot(ln < npl && rank == pos);
      if (hit) pos = (int)__builtin_ctzll(hit);
    }
  }
  const int pair = xcd + kXcds * pos, item = wi % per;
  if (pair >= p.B * p.Hkv) return;  // padding of the last round
  const int b = pair / p.Hkv, hk = pair % p.Hkv;
  const int g0 = (item % nhg) * hh;
  const int hcount = min(hh, p.G - g0);
  const int pw0 = 16 * tpw * (item / nhg);  // first row of the workgroup's tiles
  const int r0 = cu_q[b];
  const int ql = cu_q[b + 1] - r0;
  const bool first = item == 0 && hk == 0 && tid == 0;  // one report per sequence
  // rows beyond the grid would be left unwritten: report
  if (first && p.status && (ql < 0 || ql > 16 * ntiles)) atomicOr(p.status, kStatusBadSeqlen);
  if (pw0 >= ql) return;  // the whole workgroup
  if (tid == 0) s_redo = 0;  // visible after the first tile's barrier
  const int L = clamped_len(p, b, first);
  const int plast = min(pw0 + 16 * tpw - 1, ql - 1);
  const int kend = causal ? min(L, max(0, L - ql + plast + 1)) : L;  // the last tile's
  // chunks [c0, nch) of the key tiles: all of them, or the first half of the
  // tiles (rounded up) or the rest
  int c0 = 0, nch = (kend + 15) >> 4;
  if (sp >= 0) {
    const int th = ((nch + CPT - 1) / CPT + 1) >> 1;
    if (sp == 0)
      nch = min(nch, CPT * th);
    else
      c0 = CPT * th;
  }

  // slot j of this wave: unit u = w + NW j, tile u / hh, head u % hh. Column r
  // is query position p0s + r of the sequence; its keys are [0, kend_r).
  bool hon[HPW], col_ok[HPW];
  int kend_r[HPW], p0s[HPW], hls[HPW];
  // kfull[j]: the least key end over slot j's valid columns (the whole wave
  // agrees); a 32-token tile ending at or below it needs no mask
  int kfull[HPW];
  // kQ1: Q' = sign(scale) q (exact) and the scores are scaled by qmul in fp32;
  // else Q' = q scale log2 e in hi + lo parts and qmul = 1
  const float qmul = kQ1 ? (p.qscale != 0.f ? fabsf(p.qscale) : 1.f) : 1.f;
  const float qfac = kQ1 ? (p.qscale > 0.f ? 1.f : p.qscale < 0.f ? -1.f : 0.f) : p.qscale;
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
        const float y = col_ok[j] ? x[k] * qfac : 0.f;
        const T hh = (T)y;
        qhi[j][ks][k] = hh;
        if constexpr (!kQ1) qlo[j][ks][k] = (T)(y - (float)hh);
      }
    }
  }

  // The pieces this thread loads: a chunk's K or V rows are 16 x D / 8
  // 16-byte pieces, piece 64 (wh PPT + k) + lane taken by wave wh of one half
  // of the workgroup. The two halves swap K and V from one chunk to the next,
  // so every wave builds one buffer descriptor per chunk and loads (and, for
  // bf16, converts) V every other chunk.
  const int bsm = (1 << p.bs_log2) - 1;
  const int kst_bytes = (int)(p.kst * (int)sizeof(T)), vst_bytes = (int)(p.vst * (int)sizeof(T));
  const int64_t ksb_bytes = p.ksb * (int64_t)sizeof(T), vsb_bytes = p.vsb * (int64_t)sizeof(T);
  const int wh = w % (NW / 2);
  const bool vodd = w < NW / 2;  // this half loads V of the odd chunks, K of the even ones
  auto chunk_is_v = [&](int cn) -> bool { return vodd == ((cn & 1) != 0); };
  int poffk[PPT], poffv[PPT], plds[PPT];
#pragma unroll
  for (int k = 0; k < PPT; ++k) {
    const int jj = 64 * (wh * PPT + k) + lane;
    const int row = jj / (D / 8), cc = jj % (D / 8);
    poffk[k] = row * kst_bytes + 16 * cc;
    poffv[k] = row * vst_bytes + 16 * cc;
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
  int bad_block = 0;
  // (the lambdas are forced inline: called out of line, their ring arguments
  // would live in scratch memory)
  // descriptor of chunk cn's K or V rows for (validated) block id, empty for
  // id < 0
  auto chunk_rsrc = [&](int cn, int id, bool isv) __attribute__((always_inline)) {
    const int tok0 = 16 * cn;
    const int rows = id >= 0 ? min(16, kend - tok0) : 0;
    const int row0 = id >= 0 ? tok0 & bsm : 0;
    const int64_t idc = id >= 0 ? (int64_t)id : 0;
    const int st = isv ? vst_bytes : kst_bytes;
    return uniform_rsrc((isv ? vbase : kbase) + idc * (isv ? vsb_bytes : ksb_bytes) +
                            (int64_t)row0 * st,
                        rows * st);
  };
  // load this wave's pieces of chunk cn into pc; ids: the chunk's block id on
  // entry, then the id of chunk cn + NBUF
  auto issue = [&](int cn, uint4 (&pc)[PPT], int& ids) __attribute__((always_inline)) {
    int id = __builtin_amdgcn_readfirstlane(ids);
    if (cn >= nch) {
      id = -1;
    } else if (id < 0 || id >= p.NB) {
      bad_block = 1;
      id = -1;
    }
    const bool isv = chunk_is_v(cn);
    const __amdgpu_buffer_rsrc_t rs = chunk_rsrc(cn, id, isv);
#pragma unroll
    for (int k = 0; k < PPT; ++k) pc[k] = buf_load<0>(rs, isv ? poffv[k] : poffk[k]);
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

  // fold 32-token tile tc (tokens 32 tc .., staged in LDS tile `buf` from
  // element `base` on) into
  // head slot j; WIDE: the V tile holds bf16 (the second pass). P^T k-slot i of
  // lane (q, r) holds token 16 (i / 4) + 4 q + i % 4, the score MFMA's output
  // layout of the two halves.
  auto consume = [&](int tc, int buf, int base, int j, auto WIDE) __attribute__((always_inline)) {
    constexpr bool wide = decltype(WIDE)::value;
    const uint16_t* sk = s_k[buf] + base;
    const uint16_t* sv_ = s_v[buf] + base;
    f32x4 st[2] = {f32x4{0.f, 0.f, 0.f, 0.f}, f32x4{0.f, 0.f, 0.f, 0.f}};
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) {
#pragma unroll
      for (int tau = 0; tau < 2; ++tau) {
        const V8 a = *(const V8*)(sk + tau * kHalf + TR::row(r) + 8 * (4 * ks + q));
        st[tau] = M::mma32(a, qhi[j][ks], st[tau]);
        if constexpr (!kQ1) st[tau] = M::mma32(a, qlo[j][ks], st[tau]);
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
    const float mt = quad_max(mx) * qmul;
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
    for (int i = 0; i < 8; ++i) pv[i] = exp2_fast(fmaf(sv[i], qmul, -mu));
    const int vbase = TR::row(4 * q + tj) + 8 * (tk >> 1) + 4 * (tk & 1);
    // P in fp16 against the fp16 V tile, or in bf16 hi + lo parts against a
    // tile staged as bf16 (two separate loops: a branch inside one would keep
    // each 16-dim block's LDS reads from being issued ahead of its MFMA)
    H8 ph;
    V8 phi, plo;
    if constexpr (kBf && wide) {
      l[j] += ((pv[0] + pv[1]) + (pv[2] + pv[3])) + ((pv[4] + pv[5]) + (pv[6] + pv[7]));
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        const T hh = (T)pv[i];
        phi[i] = hh;
        plo[i] = (T)(pv[i] - (float)hh);
      }
    } else {
#pragma unroll
      for (int i = 0; i < 8; ++i) ph[i] = (_Float16)pv[i];
#pragma unroll
      for (int i = 0; i < 4; ++i)
        l[j] = __builtin_amdgcn_fdot2(h2{ph[2 * i], ph[2 * i + 1]}, h2{1, 1}, l[j], false);
    }
    if constexpr (kBf && wide) {
#pragma unroll
      for (int mb = 0; mb < MB; ++mb) {
        const int o = vbase + 16 * mb;
        const s16x4 lo4 = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4*)(sv_ + o));
        const s16x4 hi4 = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4*)(sv_ + kHalf + o));
        const V8 av = __builtin_bit_cast(V8, __builtin_shufflevector(lo4, hi4, 0, 1, 2, 3, 4, 5, 6, 7));
        acc[j][mb] = M::mma32(av, phi, acc[j][mb]);
        acc[j][mb] = M::mma32(av, plo, acc[j][mb]);
      }
    } else {
#pragma unroll
      for (int mb = 0; mb < MB; ++mb) {
        const int o = vbase + 16 * mb;
        const s16x4 lo4 = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4*)(sv_ + o));
        const s16x4 hi4 = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4*)(sv_ + kHalf + o));
        const H8 av = __builtin_bit_cast(H8, __builtin_shufflevector(lo4, hi4, 0, 1, 2, 3, 4, 5, 6, 7));
        acc[j][mb] = H::mma32(av, ph, acc[j][mb]);
      }
    }
  };

  // all of the wave's head slots against tile tc (V in fp16), each K and V^T
  // fragment read from LDS once for all of them (a wave's units share the
  // workgroup's keys): half the fragment reads per MFMA of one slot at a time
  auto consume_all = [&](int tc, int buf, int base) __attribute__((always_inline)) {
    const uint16_t* sk = s_k[buf] + base;
    const uint16_t* sv_ = s_v[buf] + base;
    f32x4 st[HPW][2];
#pragma unroll
    for (int j = 0; j < HPW; ++j) st[j][0] = st[j][1] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) {
#pragma unroll
      for (int tau = 0; tau < 2; ++tau) {
        const V8 a = *(const V8*)(sk + tau * kHalf + TR::row(r) + 8 * (4 * ks + q));
#pragma unroll
        for (int j = 0; j < HPW; ++j) {
          st[j][tau] = M::mma32(a, qhi[j][ks], st[j][tau]);
          if constexpr (!kQ1) st[j][tau] = M::mma32(a, qlo[j][ks], st[j][tau]);
        }
      }
    }
    H8 ph[HPW];
#pragma unroll
    for (int j = 0; j < HPW; ++j) {
      float sv[8];
      if (32 * tc + 32 <= kfull[j]) {
#pragma unroll
        for (int i = 0; i < 8; ++i) sv[i] = st[j][i >> 2][i & 3];
      } else {
#pragma unroll
        for (int i = 0; i < 8; ++i)
          sv[i] = (32 * tc + 16 * (i >> 2) + 4 * q + (i & 3) < kend_r[j]) ? st[j][i >> 2][i & 3]
                                                                          : -INFINITY;
      }
      float mx = sv[0];
#pragma unroll
      for (int i = 1; i < 8; ++i) mx = fmaxf(mx, sv[i]);
      const float mt = quad_max(mx) * qmul;
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
#pragma unroll
      for (int i = 0; i < 8; ++i) ph[j][i] = (_Float16)exp2_fast(fmaf(sv[i], qmul, -mu));
#pragma unroll
      for (int i = 0; i < 4; ++i)
        l[j] = __builtin_amdgcn_fdot2(h2{ph[j][2 * i], ph[j][2 * i + 1]}, h2{1, 1}, l[j], false);
    }
    const int vbase = TR::row(4 * q + tj) + 8 * (tk >> 1) + 4 * (tk & 1);
#pragma unroll
    for (int mb = 0; mb < MB; ++mb) {
      const int o = vbase + 16 * mb;
      const s16x4 lo4 = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4*)(sv_ + o));
      const s16x4 hi4 = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4*)(sv_ + kHalf + o));
      const H8 av = __builtin_bit_cast(H8, __builtin_shufflevector(lo4, hi4, 0, 1, 2, 3, 4, 5, 6, 7));
#pragma unroll
      for (int j = 0; j < HPW; ++j) acc[j][mb] = H::mma32(av, ph[j], acc[j][mb]);
    }
  };

  // One pass over the workgroup's tiles [c0, nch) (WIDE: V staged as bf16). The ring:
  // chunk c + NBUF - 1 is issued just before chunk c is staged
  // (unconditionally: past the end the descriptors are empty, so a short
  // last tile is filled up with zeros). Chunk c goes to part c % CPT of LDS
  // tile (c / CPT) % 2; the barrier after a tile's last part also means every
  // wave is done with the tile before, so the other tile is free.
  const int nch2 = (nch + CPT - 1) / CPT * CPT;
  auto fold_all = [&](auto WIDE) __attribute__((always_inline)) {
    constexpr bool wide = decltype(WIDE)::value;
    int idr[NBUF];
    static_for<0, NBUF>([&](auto S) { idr[decltype(S)::value] = fetch_id(c0 + decltype(S)::value); });
    uint4 ring[NBUF][PPT];
    static_for<0, NBUF - 1>([&](auto S) {
      constexpr int s = decltype(S)::value;
      issue(c0 + s, ring[s], idr[s]);
    });
    for (int cb = c0; cb < nch2; cb += NBUF) {
      static_for<0, NBUF>([&](auto S) {
        constexpr int s = decltype(S)::value;
        constexpr int sn = (s + NBUF - 1) % NBUF;
        const int c = cb + s;
        issue(c + NBUF - 1, ring[sn], idr[sn]);
        __builtin_amdgcn_sched_barrier(0);
        if (c < nch2) {
          const int buf = (c / CPT) & 1, half = (c % CPT) * kHalf;
          const bool isv = chunk_is_v(c);
#pragma unroll
          for (int k = 0; k < PPT; ++k) {
            uint4 x = ring[s][k];
            if constexpr (kBf && !wide) {
              if (isv) x = bf16x8_to_f16(x);
            }
            *(uint4*)((isv ? s_v[buf] : s_k[buf]) + half + plds[k]) = x;
          }
          if (c % CPT == CPT - 1) {
            __syncthreads();
#pragma unroll
            for (int st = 0; st < CPT / 2; ++st) {
              const int tc = (c >> 1) - (CPT / 2 - 1) + st;
              if constexpr (HPW > 1 && !wide) {
                consume_all(tc, buf, 2 * st * kHalf);  // (a slot without a unit folds zeros, unread)
              } else {
#pragma unroll
                for (int j = 0; j < HPW; ++j)
                  if (hon[j]) consume(tc, buf, 2 * st * kHalf, j, WIDE);
              }
            }
          }
        }
      });
    }
  };
  fold_all(std::false_type());
  if constexpr (kBf) {
    // a bf16 V value beyond fp16's range (or a non-finite input) left a
    // non-finite output: fold every tile again with V as bf16
    bool bad = false;
#pragma unroll
    for (int j = 0; j < HPW; ++j)
#pragma unroll
      for (int mb = 0; mb < MB; ++mb)
#pragma unroll
        for (int e = 0; e < 4; ++e) bad = bad || !__builtin_isfinite(acc[j][mb][e]);
    if (__ballot(bad) && lane == 0) s_redo = 1;
    __syncthreads();
    if (__builtin_amdgcn_readfirstlane(s_redo)) {
#pragma unroll
      for (int j = 0; j < HPW; ++j) {
#pragma unroll
        for (int k = 0; k < MB; ++k) acc[j][k] = f32x4{0.f, 0.f, 0.f, 0.f};
        m[j] = -INFINITY;
        l[j] = 0.f;
      }
      fold_all(std::true_type());
    }
  }

  if (sp >= 0) {
    // Key split: store this half's state per unit u = w + NW j (output
    // fragments in lane order, then m and l per lane), count in, and let the
    // second half to arrive merge the first's state into its own.
    constexpr int US = MB * 256 + 128;  // floats per unit and half
    const int64_t si = (int64_t)xcd * nsplit + (wi - nwhole);
    const __amdgpu_buffer_rsrc_t rst_ = uniform_rsrc((const char*)(ws_st + si * (2 * 8 * US)),
                                                     2 * 8 * US * 4);
#pragma unroll
    for (int j = 0; j < HPW; ++j) {
      const int o = (sp * 8 + w + NW * j) * US;
#pragma unroll
      for (int mb = 0; mb < MB; ++mb)
        __builtin_amdgcn_raw_buffer_store_b128(__builtin_bit_cast(u32x4, acc[j][mb]), rst_,
                                               (o + (mb * 64 + lane) * 4) * 4, 0, kScDevice);
      __builtin_amdgcn_raw_buffer_store_b32(__float_as_uint(m[j]), rst_,
                                            (o + MB * 256 + lane) * 4, 0, kScDevice);
      __builtin_amdgcn_raw_buffer_store_b32(__float_as_uint(l[j]), rst_,
                                            (o + MB * 256 + 64 + lane) * 4, 0, kScDevice);
    }
    // Ordering: the stores are device scope, so they complete at the
    // device-coherent level; every wave waits for its own (the signal fences
    // keep the compiler from moving memory operations across the wait) before
    // the barrier, and only then does one thread count the workgroup in with an
    // agent-scope atomic. The two increments of a counter are ordered at its
    // point of coherence, so the half that reads 1 counts in after the other
    // half's states were complete; its loads below depend on that value and
    // are device scope as well.
    __atomic_signal_fence(__ATOMIC_SEQ_CST);
    __builtin_amdgcn_s_waitcnt(0);
    __atomic_signal_fence(__ATOMIC_SEQ_CST);
    __syncthreads();
    if (tid == 0)
      s_arrived = __hip_atomic_fetch_add(ws_cnt + si, 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    __syncthreads();
    if (__builtin_amdgcn_readfirstlane(s_arrived) == 0) return;  // the other half merges
    // second to arrive: reset the counter for the next call (the kernel
    // boundary orders this store before any later launch)
    if (tid == 0) __hip_atomic_store(ws_cnt + si, 0, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    __atomic_signal_fence(__ATOMIC_SEQ_CST);
#pragma unroll
    for (int j = 0; j < HPW; ++j) {
      const int o = ((1 - sp) * 8 + w + NW * j) * US;
      const float mo = __uint_as_float(
          __builtin_amdgcn_raw_buffer_load_b32(rst_, (o + MB * 256 + lane) * 4, 0, kScDevice));
      const float lo = __uint_as_float(
          __builtin_amdgcn_raw_buffer_load_b32(rst_, (o + MB * 256 + 64 + lane) * 4, 0, kScDevice));
      const float M = fmaxf(m[j], mo);
      const float mu = M == -INFINITY ? 0.f : M;
      const float w0 = exp2_fast(m[j] - mu), w1 = exp2_fast(mo - mu);
      l[j] = w0 * l[j] + w1 * lo;
      m[j] = M;
#pragma unroll
      for (int mb = 0; mb < MB; ++mb) {
        const f32x4 ao = __builtin_bit_cast(
            f32x4, __builtin_amdgcn_raw_buffer_load_b128(rst_, (o + (mb * 64 + lane) * 4) * 4, 0,
                                                         kScDevice));
        acc[j][mb] = w0 * acc[j][mb] + w1 * ao;
      }
    }
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

// {waves per workgroup, ring slots, waves per SIMD} per Q' form and head_dim.
// Q' forms: 0 fp32 q (two parts), 1 bf16 q over fp16 K/V (two parts), 2 bf16 q
// over bf16 K/V (one exact part). At d = 128 four waves of two units each
// (their K and V^T fragments read once for both): two workgroups per compute
// unit with fp32 q, three with one Q' part; bf16 q over fp16 K/V keeps eight
// waves of one unit.
constexpr int kPrefillCfg[3][3][3] = {{{4, 6, 2}, {4, 4, 2}, {8, 4, 2}},
                                      {{4, 6, 2}, {8, 4, 4}, {8, 4, 2}},
                                      {{4, 6, 2}, {4, 2, 3}, {8, 4, 2}}};
constexpr int pdim(int D) { return D == 64 ? 0 : D == 128 ? 1 : 2; }
constexpr int qform(int dtype, int qo) { return qo == 0 ? 0 : dtype == 2 ? 2 : 1; }

// The launch's shape: heads per workgroup, work items per (sequence, KV head)
// and per XCD, and how many of each XCD's items are whole and split.
struct Plan {
  int hh = 8, nhg = 1, ntiles = 0, per = 0;
  int64_t items = 0;  // per XCD (the last round of pairs padded)
  int64_t nwhole = 0, nsplit = 0;
  int D = 0;
};

Plan plan(const Params& p, int dtype, int max_q) {
  Plan pl;
  const int qf = qform(dtype, p.qo_bf16 ? 1 : 0), di = pdim(p.D);
  const int NW = kPrefillCfg[qf][di][0], OCC = kPrefillCfg[qf][di][2];
  pl.D = p.D;
  // heads per workgroup: 8 when they divide G; else the largest power of two
  // dividing G, with 8 / hh tiles per workgroup so that no unit is idle, if
  // there are that many tiles (else 8, the last group partly empty)
  pl.ntiles = (max_q + 15) / 16;
  pl.hh = kHeadsPerGroup;
  if (p.G % kHeadsPerGroup) {
    int h2 = 1;
    while (2 * h2 < kHeadsPerGroup && p.G % (2 * h2) == 0) h2 *= 2;
    if (pl.ntiles >= kHeadsPerGroup / h2) pl.hh = h2;
  }
  const int tpw = kHeadsPerGroup / pl.hh;
  pl.nhg = (p.G + pl.hh - 1) / pl.hh;
  // per (sequence, KV head): tile groups x head groups; pairs spread over the
  // XCDs, the last round padded with empty workgroups
  pl.per = (pl.ntiles + tpw - 1) / tpw * pl.nhg;
  const int64_t rounds = ((int64_t)p.B * p.Hkv + kXcds - 1) / kXcds;
  pl.items = rounds * pl.per;
  pl.nwhole = pl.items;
  // the key split: an XCD holds C workgroups at once; when its items leave a
  // last round at most half full, that round's items run as two halves each
  const int64_t C = (int64_t)(p.cus / kXcds) * (4 * OCC / NW);
  if (C > 0) {
    const int64_t k = pl.items / C, rem = pl.items - k * C;
    if (k >= 1 && rem > 0 && 2 * rem <= C) {
      pl.nwhole = k * C;
      pl.nsplit = rem;
    }
  }
  return pl;
}

// floats of one split item's two halves' states: 8 units x (D / 16 output
// fragments of 64 lanes x 4, then m and l of 64 lanes)
int64_t split_item_floats(int D) { return 2 * 8 * ((int64_t)(D / 16) * 256 + 128); }
size_t split_cnt_bytes(const Plan& pl) {
  return ((size_t)kXcds * pl.nsplit * sizeof(int32_t) + 255) & ~(size_t)255;
}

template <typename T, int D, int QO>
hipError_t launch_p(const Params& p, const int32_t* cu_q, int max_q, int causal, void* ws,
                    hipStream_t s) {
  constexpr int QF = qform(std::is_same<T, __bf16>::value ? 2 : 1, QO);
  constexpr int NW = kPrefillCfg[QF][pdim(D)][0], NB_ = kPrefillCfg[QF][pdim(D)][1],
                OCC = kPrefillCfg[QF][pdim(D)][2];
  Plan pl = plan(p, std::is_same<T, __bf16>::value ? 2 : 1, max_q);
  if (!ws) {
    pl.nwhole = pl.items;
    pl.nsplit = 0;
  }
  const int64_t blocks = kXcds * (pl.nwhole + 2 * pl.nsplit);
  if (blocks > 0x7fffffff || pl.items > 0x3fffffff) return hipErrorInvalidConfiguration;
  int32_t* cnt = pl.nsplit > 0 ? (int32_t*)ws : nullptr;
  float* st = pl.nsplit > 0 ? (float*)((char*)ws + split_cnt_bytes(pl)) : nullptr;
  hipLaunchKernelGGL((prefill_kernel<T, D, NW, NB_, OCC, QO>), dim3((unsigned)blocks),
                     dim3(64 * NW), 0, s, p, cu_q, causal, pl.nhg, pl.hh, pl.ntiles, pl.per,
                     (int)pl.nwhole, (int)pl.nsplit, cnt, st);
  return hipGetLastError();
}

template <typename T>
hipError_t launch_pd(const Params& p, const int32_t* cu_q, int max_q, int causal, void* ws,
                     hipStream_t s) {
  const bool bf = p.qo_bf16 != 0;
  switch (p.D) {
    case 64: return bf ? launch_p<T, 64, 1>(p, cu_q, max_q, causal, ws, s)
                       : launch_p<T, 64, 0>(p, cu_q, max_q, causal, ws, s);
    case 128: return bf ? launch_p<T, 128, 1>(p, cu_q, max_q, causal, ws, s)
                        : launch_p<T, 128, 0>(p, cu_q, max_q, causal, ws, s);
    case 256: return bf ? launch_p<T, 256, 1>(p, cu_q, max_q, causal, ws, s)
                        : launch_p<T, 256, 0>(p, cu_q, max_q, causal, ws, s);
  }
  return hipErrorInvalidValue;
}

}  // namespace

hipError_t launch_prefill(const Params& p, int dtype, const int32_t* cu_q, int max_q, int causal,
                          void* ws, hipStream_t s) {
  if (max_q <= 0 || p.B <= 0) return hipSuccess;
  if (dtype == 1) return launch_pd<_Float16>(p, cu_q, max_q, causal, ws, s);
  if (dtype == 2) return launch_pd<__bf16>(p, cu_q, max_q, causal, ws, s);
  return hipErrorInvalidValue;
}

size_t prefill_workspace_bytes(const Params& p, int dtype, int max_q) {
  if (max_q <= 0 || p.B <= 0 || (p.D != 64 && p.D != 128 && p.D != 256)) return 0;
  const Plan pl = plan(p, dtype, max_q);
  if (pl.nsplit == 0) return 0;
  return split_cnt_bytes(pl) + (size_t)kXcds * pl.nsplit * split_item_floats(p.D) * sizeof(float);
}

size_t prefill_workspace_zeroed_bytes(const Params& p, int dtype, int max_q) {
  if (prefill_workspace_bytes(p, dtype, max_q) == 0) return 0;
  return (size_t)kXcds * plan(p, dtype, max_q).nsplit * sizeof(int32_t);
}

}  // namespace pa
