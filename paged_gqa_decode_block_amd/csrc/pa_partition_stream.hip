// pa_partition_stream.hip -- persistent streaming partition kernel (MFMA, gfx950).
//
// The split-KV decomposition (page "Paged Attention Kernel Architecture for
// BI-V100", sections 4 and 6) is counted in 16-token chunks: each (sequence b,
// KV head) token stream has ceil(L_b / 16) of them, numbered sequence by
// sequence, KV head by KV head. Two waves per SIMD (by default) are launched
// (a multiple of the compute-unit count) and the waves in use take equal
// contiguous shares of the chunks, so every compute unit streams the same number
// of bytes. A share mostly walks one stream. Along a stream the wave keeps a
// ring of NBUF 16-token chunks of K and V in flight in registers; the ring's
// issue is unconditional and its table reads travel in ring order, so the wait
// before each chunk covers that chunk's loads only.
//
// At head_dim 256 a share belongs to a pair of waves (one workgroup) that split
// the head dims: each loads, stages and folds 128 of them, and their partial
// scores meet in LDS once per chunk (one barrier), so both keep the same
// softmax state while each holds half of the output. That keeps a wave at
// d = 128's registers and two waves per SIMD, so one wave's folding overlaps
// the other's loads.
//
// The split of the KV sequence is the waves' shares themselves (the partition
// size is not used): a stream that lies inside one share is folded whole and
// its normalised output written directly; a stream that several consecutive
// waves share leaves one partial state (max, sum, unnormalised output) per
// wave, written once when the wave's segment of it ends (the share's first
// segment's state, when more segments follow, waits in LDS until the share
// ends: a store in the middle of the share would make the next chunk's wait
// cover it), and the combine kernel merges those states. A share partly covers at most two streams (its
// first and its last), so each wave has two state slots; the wave holding a
// stream's first chunk records which slot starts the stream's run of states
// and how many waves the run spans. Writing one state per wave, not one per
// fixed-size partition, keeps the bytes written small: on the 64-sequence
// batch about half of what 4096-token partitions plus continuation pieces
// wrote, and those writes cost far more time than their share of the traffic.
//
// Loads are raw buffer loads of full token rows (each 16-byte lane load is part
// of a contiguous row segment of 128-512 bytes) with the non-temporal hint,
// except where blocks are declared shared: there the folded prefixes keep the
// default policy (several groups read them) and, without folding, every load
// does. The per-chunk buffer descriptor (built in scalar registers) starts at the chunk's
// first row and its size covers only the attended rows, so rows past L_b and
// chunks behind an invalid table entry read as zeros without touching memory.
// Each chunk is then written to two padded LDS tiles and read back in MFMA
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
// it by more than 8, so p <= 256 and most chunks skip the rescale. At the end
// of each of the share's segments the state is written (a state slot, or the
// normalised output when the segment is a whole stream). Tokens at or past L_b
// and chunks behind an invalid table entry are never loaded; their scores are
// -inf.
//
// Prefix folding (blocks declared shared): sequences are taken in groups of F
// = 16 / G, and the streams become those of virtual sequences: per group its
// folded prefix (the leading blocks every member lists and attends whole,
// found by fold_scan_kernel), read through the first member's table with the
// F x G (member, head) pairs as the score MFMA's 16 columns (the padding the
// G heads alone leave), then each member's tokens past the prefix. Neither
// kind is written out: a stream inside one share leaves its one state in its
// own rows, a shared one a state per wave as above, and the combine merges a
// sequence's own states with its column of the group's prefix states. The
// prefix is read once per group instead of once per member.
//
// Requires block_size >= 16 (a 16-token chunk lies in one block), at most 1024
// (virtual) sequences (the chunk prefix is formed in registers) and fewer than
// 2^31 chunks per KV head in the batch.
#include <type_traits>

#include "pa_mfma_util.h"

namespace pa {
namespace {

constexpr int kMaxWindows = 16;  // 16 x 64 = 1024 sequences

// Partial-state stores. wt: with the device-scope cache policy (SC1 set, SC0
// clear on gfx950), written through the XCD's L2 as they are made rather than
// left dirty there for the write-back at the kernel's end (the combine kernel
// reads them from the other XCDs anyway). On the one-wave-per-share kernel
// without prefix folding, whose waves end over a wide spread of times, that
// measured faster (64-sequence batch, partition kernel -3 us); where the
// waves end together (pairs at head_dim 256) or with prefix folding it
// measured slower, so those keep the default policy. The store takes the
// same per-lane address registers as a plain one (no buffer descriptor held
// in the loop).
__device__ __forceinline__ void store_state4(float* ptr, f32x4 v, bool wt) {
  if (wt)
    asm volatile("global_store_dwordx4 %0, %1, off sc1" : : "v"(ptr), "v"(v) : "memory");
  else
    *(f32x4*)ptr = v;
}
__device__ __forceinline__ void store_state1(float* ptr, float v, bool wt) {
  if (wt)
    asm volatile("global_store_dword %0, %1, off sc1" : : "v"(ptr), "v"(v) : "memory");
  else
    *ptr = v;
}

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
// allocation is held to. POL: cache policy of the K/V loads. DS: waves sharing
// one share (1, or 2: a workgroup of two waves splits the head dims, each
// loading, staging and folding D / 2 of them; their partial scores are added
// through LDS once per chunk, so both hold the same softmax state).
template <typename T, int D, int NBUF, int OCC, int POL, bool QL, int QO, int DS>
__global__ void __launch_bounds__(64 * DS) __attribute__((amdgpu_waves_per_eu(OCC, OCC)))
partition_stream_kernel(Params p) {
  typedef Mx<T> M;
  typedef typename M::v8 V8;
  typedef typename M::v4 V4;
  constexpr int DW = D / DS;  // head dims this wave loads and folds
  typedef Cfg<DW> C;
  constexpr int LPC = C::LPC, KS = C::KS, MB = C::MB;
  static_assert(DS == 1 || DS == 2, "one wave or a pair per share");
  static_assert((NBUF - 1) * 2 * LPC <= 63, "ring deeper than the vector-memory counter");

  constexpr bool kQLds = QL;  // Q' fragments in LDS (else in registers)
  typedef TileRows<DW> TR;  // padded K and V tiles (bank-conflict free reads)
  __shared__ __attribute__((aligned(16))) uint16_t s_k[DS][TR::SIZE];
  __shared__ __attribute__((aligned(16))) uint16_t s_v[DS][TR::SIZE];
  __shared__ __attribute__((aligned(16))) V8 s_q[DS][kQLds ? 2 : 1][kQLds ? KS : 1][64];
  // partial scores of the pair, double-buffered by chunk parity
  __shared__ __attribute__((aligned(16))) f32x4 s_x[DS == 2 ? 2 : 1][DS][64];
  // the share's first segment's partial state while later segments stream
  // (stored at the share's end: a store in the middle would make the next
  // chunk's wait cover it)
  __shared__ __attribute__((aligned(16))) f32x4 s_park[DS][MB][64];
  __shared__ float s_park_ml[DS][2][64];

  const int lane = threadIdx.x & 63;
  // which half of the head dims this wave holds (0 when DS = 1), uniform
  const int half = DS == 2 ? __builtin_amdgcn_readfirstlane((int)(threadIdx.x >> 6)) : 0;
  int par = 0;  // chunk parity of the score exchange
  const int r = lane & 15, q = lane >> 4;
  const int G = p.G, Hkv = p.Hkv;

  // ---- 1. chunk counts and this wave's share ---------------------------------
  // Work is counted in 16-token chunks: sequence b has nc(b) = ceil(L_b / 16)
  // chunks per KV head, numbered sequence by sequence, KV head by KV head,
  // token by token. The waves in use take equal contiguous shares (sizes at
  // most one chunk apart), and their number is a multiple of the compute-unit
  // count whenever there is enough work, so every compute unit streams the
  // same number of bytes until the end. A share may begin or end inside a
  // partition; the wave then leaves that piece as a continuation state.
  // All windows' lengths are loaded before any is checked, so the loads travel
  // together; wave 0 reports an out-of-range length once.
  //
  // With prefix folding the streams are those of virtual sequences: group i
  // (sequences F i .. F i + F - 1) is virtual sequences (F + 1) i (its folded
  // prefix, read through the first member's table) and (F + 1) i + 1 + m
  // (member m's own tokens past the prefix), whose lengths the fold scan left
  // in p.ws_vlen (and which reported any out-of-range length).
  const int F = p.fold;
  const int nv = F > 0 ? (p.B + F - 1) / F * (F + 1) : p.B;
  const int nwin = (nv + 63) >> 6;
  int ncw[kMaxWindows], lw[kMaxWindows];
  int tot = 0;
#pragma unroll
  for (int wi = 0; wi < kMaxWindows; ++wi) {
    const int v = wi * 64 + lane;
    lw[wi] = (wi < nwin && v < nv) ? (F > 0 ? p.ws_vlen[v] : p.seqlens[v]) : 0;
  }
  {
    const int lmax = p.MBS << p.bs_log2;
    bool bad_len = false;
#pragma unroll
    for (int wi = 0; wi < kMaxWindows; ++wi) {
      const int v = wi * 64 + lane;
      int Lb = lw[wi] + (F > 0 ? 0 : p.len_add);
      if (wi < nwin && v < nv && (Lb < 0 || Lb > lmax)) {
        bad_len = true;
        Lb = Lb < 0 ? 0 : lmax;
      }
      lw[wi] = (wi < nwin && v < nv) ? Lb : 0;
      ncw[wi] = (lw[wi] + 15) >> 4;
    }
    if (blockIdx.x == 0 && __ballot(bad_len) && lane == 0 && p.status)
      atomicOr(p.status, kStatusBadSeqlen);
  }
  {
    // lane-local sum over the windows, then one wave reduction
    int s = 0;
#pragma unroll
    for (int wi = 0; wi < kMaxWindows; ++wi) s += ncw[wi];
#pragma unroll
    for (int off = 32; off >= 1; off >>= 1) s += __shfl_xor(s, off);
    tot = s;  // uniform
  }
  // 32-bit chunk arithmetic: the host admits only batches with fewer than
  // 2^31 chunks. Wave x takes base + (x < extra) chunks starting at
  // x * base + min(x, extra).
  const int n_chunks = tot * Hkv;
  const int nw = stream_active_waves32(n_chunks, (int)gridDim.x, p.cus);
  if ((int)blockIdx.x >= nw) return;
  const int sh_base = n_chunks / nw, sh_extra = n_chunks - sh_base * nw;
  const int wx = (int)blockIdx.x;
  int g = wx * sh_base + min(wx, sh_extra);
  const int g_end = g + sh_base + (wx < sh_extra ? 1 : 0);
  if (g >= g_end) return;

  // (virtual) sequence holding chunk g: Hkv * P(v) <= g < Hkv * P(v + 1), P =
  // prefix of nc; L is the stream's length in tokens
  int b = 0, ncb = 1, L = 0;
  int Pb = 0;
  {
    const int x = g / Hkv;
    int carry = 0;
    bool found = false;
#pragma unroll
    for (int wi = 0; wi < kMaxWindows; ++wi) {
      if (!found && wi < nwin) {
        const int incl = wave_incl_scan(ncw[wi], lane) + carry;
        const uint64_t hit = __ballot(incl > x && ncw[wi] > 0);
        if (hit) {
          const int src = __builtin_ctzll(hit);
          b = wi * 64 + src;  // the virtual sequence, resolved below
          ncb = __shfl(ncw[wi], src);
          L = __shfl(lw[wi], src);
          Pb = __shfl(incl, src) - ncb;
          found = true;
        }
        carry = __shfl(incl, 63);
      }
    }
  }
  int hk, j;
  {
    const int e = g - Pb * Hkv;
    hk = e / ncb;
    j = e - hk * ncb;
  }
  // virtual sequence v: its table row b, first token toff, and whether it is
  // a group's folded prefix (fseg, group gi, members nm); set by resolve(v)
  int v = b, toff = 0, gi = 0, nm = 1;
  bool fseg = false;

  const int bsm = (1 << p.bs_log2) - 1;
  const int rowL = lane / C::CPR;  // row within a load instruction
  const int cc = lane % C::CPR;    // 16-byte chunk of the row this lane loads
  const int tj = r >> 2, tk = r & 3;

  // byte offsets of this lane's 16-byte piece of row s*RPI + rowL in a chunk
  const int kst_bytes = (int)(p.kst * (int)sizeof(T)), vst_bytes = (int)(p.vst * (int)sizeof(T));
  const int hoff = half * DW * (int)sizeof(T);  // this wave's dims within a row
  int koffs[LPC], voffs[LPC];
#pragma unroll
  for (int s = 0; s < LPC; ++s) {
    koffs[s] = (s * C::RPI + rowL) * kst_bytes + 16 * cc + hoff;
    voffs[s] = (s * C::RPI + rowL) * vst_bytes + 16 * cc + hoff;
  }

  // ---- 2. segments: the share's runs of chunks within one (b, KV head) -------
  int bad_block = 0;
  bool first_seg = true;
  int park_cols = 0;  // the first segment's state waits in s_park: its valid columns
  const bool wt = DS == 1 && F == 0;  // write-through partial states (store_state4)
  while (g < g_end) {
    if (F > 0) {
      gi = v / (F + 1);
      const int k = v - gi * (F + 1);
      fseg = k == 0;
      b = gi * F + (fseg ? 0 : k - 1);
      toff = fseg ? 0 : p.ws_vlen[gi * (F + 1)];
      nm = min(F, p.B - gi * F);
    } else {
      b = v;
    }
    const int jA = j;
    const int nch = min(ncb - j, g_end - g);
    const int cs = Pb * Hkv + hk * ncb;  // the stream's first chunk in the batch
    {
      const int T0 = toff + 16 * jA;
      const int T1 = toff + min(L, 16 * (jA + nch));
      const int32_t* trow = p.table + (int64_t)b * p.MBS;
      const char* kbase = (const char*)p.k + (int64_t)hk * p.ksh * (int)sizeof(T);
      const char* vbase = (const char*)p.v + (int64_t)hk * p.vsh * (int)sizeof(T);

      // Table entries of the segment's blocks, read through a descriptor over
      // exactly those entries (chunks past the end read 0 and are masked by
      // cn < nch). Each issue also fetches the entry of the chunk its ring slot
      // takes next, NBUF chunks later, so the fetch travels in ring order and
      // its wait never covers loads still in flight for later chunks.
      const int nblk = (T1 + bsm) >> p.bs_log2;
      const __amdgpu_buffer_rsrc_t rst = uniform_rsrc((const char*)trow, nblk * 4);
      auto fetch_id = [&](int cn) -> int {
        return (int)__builtin_amdgcn_raw_buffer_load_b32(rst, ((T0 + 16 * cn) >> p.bs_log2) * 4, 0, 0);
      };
      int idr[NBUF];
      static_for<0, NBUF>([&](auto S) { idr[decltype(S)::value] = fetch_id(decltype(S)::value); });
      // table entries before Q in the load queue: the ring's first issue waits
      // for the entries only
      __builtin_amdgcn_sched_barrier(0);

      // Q of head r (zero for padded heads): the loads are issued here, but
      // turned into Q' fragments only after the ring's first K/V loads are
      // issued, so the wave's first HBM requests do not wait for Q.
      // column r of the score MFMA: head r of sequence b, or in a folded
      // prefix head r % G of member r / G
      const bool hv = fseg ? (r < nm * G) : r < G;
      float4 qa[KS], qb[KS];
      {
        const int qb_ = fseg && hv ? b + r / G : b;
        const int qh = hv ? (fseg ? r % G : r) : 0;
        const int64_t qrow = ((int64_t)qb_ * p.Hq + hk * G + qh) * D + half * DW + 8 * q;
        // every lane loads (padded heads read head 0's row, a valid address)
        // and make_q zeroes padded heads: no branch around the loads
#pragma unroll
        for (int ks = 0; ks < KS; ++ks) {
          qa[ks] = load_q4<QO>(p, qrow + 32 * ks);
          qb[ks] = load_q4<QO>(p, qrow + 32 * ks + 4);
        }
      }
      V8 qhi[kQLds ? 1 : KS], qlo[kQLds ? 1 : KS];
      auto make_q = [&]() {
#pragma unroll
        for (int ks = 0; ks < KS; ++ks) {
          float x[8] = {qa[ks].x, qa[ks].y, qa[ks].z, qa[ks].w,
                        qb[ks].x, qb[ks].y, qb[ks].z, qb[ks].w};
#pragma unroll
          for (int k = 0; k < 8; ++k) x[k] = hv ? x[k] : 0.f;
          V8 hi, lo;
#pragma unroll
          for (int k = 0; k < 8; ++k) {
            const float y = x[k] * p.qscale;
            const T h = (T)y;
            hi[k] = h;
            lo[k] = (T)(y - (float)h);
          }
          if constexpr (kQLds) {
            s_q[half][0][ks][lane] = hi;
            s_q[half][1][ks][lane] = lo;
          } else {
            qhi[ks] = hi;
            qlo[ks] = lo;
          }
        }
      };

      // issue the loads of chunk cn into one ring slot; returns the chunk's
      // number of attended rows (0 behind an invalid table entry). The buffer
      // descriptors cover exactly those rows: lanes whose row lies beyond them
      // read zeros without a memory access.
      // An entry outside [0, NB) inside the attended range is never
      // dereferenced; it is noted in bad_block and reported once when the
      // wave ends (no store or atomic sits between the ring's loads).
      auto issue = [&](int cn, uint4 (&rk)[LPC], uint4 (&rv)[LPC], int& ids) -> int {
        // the entry is read whatever cn is: a read inside the cn < nch branch
        // lets the compiler move the entry's load next to it and wait for it
        // (and everything issued before) right there
        int id = __builtin_amdgcn_readfirstlane(ids);
        if (cn >= nch) {
          id = -1;
        } else if (id < 0 || id >= p.NB) {
          bad_block = 1;
          id = -1;
        }
        const int tok0 = T0 + 16 * cn;
        const int rows = id >= 0 ? min(16, T1 - tok0) : 0;
        const int64_t row0 = id >= 0 ? (int64_t)(tok0 & bsm) : 0;
        const int64_t idc = id >= 0 ? (int64_t)id : 0;
        const __amdgpu_buffer_rsrc_t rsk = uniform_rsrc(
            kbase + (idc * p.ksb + row0 * p.kst) * (int)sizeof(T), rows * kst_bytes);
        const __amdgpu_buffer_rsrc_t rsv = uniform_rsrc(
            vbase + (idc * p.vsb + row0 * p.vst) * (int)sizeof(T), rows * vst_bytes);
        // with prefix folding only the folded prefixes keep POL (their blocks
        // are read once per group, by several groups); every other segment's
        // blocks are read once in the whole launch
        if (POL == 2 || (F > 0 && !fseg)) {
#pragma unroll
          for (int s = 0; s < LPC; ++s) {
            rk[s] = buf_load<2>(rsk, koffs[s]);
            rv[s] = buf_load<2>(rsv, voffs[s]);
          }
        } else {
#pragma unroll
          for (int s = 0; s < LPC; ++s) {
            rk[s] = buf_load<POL>(rsk, koffs[s]);
            rv[s] = buf_load<POL>(rsv, voffs[s]);
          }
        }
        ids = fetch_id(cn + NBUF);
        return rows;
      };

      f32x4 acc[MB];
#pragma unroll
      for (int k = 0; k < MB; ++k) acc[k] = f32x4{0.f, 0.f, 0.f, 0.f};
      float m = -INFINITY, l = 0.f;

      // Write the segment's result once, when its last chunk is folded. A
      // segment that is the whole stream writes the normalised output. Any
      // other segment is part of a stream several consecutive waves share: it
      // leaves its state (max, sum, unnormalised output of the G heads) in
      // this wave's slot 0 when it is the share's first segment, else slot 1
      // (a share has at most one partly covered stream at each end). The wave
      // holding the stream's first chunk also names the stream's states: the
      // slot of its own state and the number of waves whose states make up
      // the stream (0 when the output was written here).
      auto flush = [&]() {
        // a stream inside this share is written out, except a folded prefix or
        // a member's stream behind one: those leave their one state in the
        // stream's own rows (with folding only); a stream that several waves
        // share leaves one state per wave in the wave's slots
        const bool inside = jA == 0 && nch == ncb;
        const bool whole = inside && !fseg && toff == 0;
        const bool own = inside && !whole;
        const int64_t rec = fseg ? (int64_t)(p.B + gi) * Hkv + hk : (int64_t)b * Hkv + hk;
        const int slot = 2 * wx + (first_seg ? 0 : 1);
        const float lt = quad_sum(l);
        if (hv) {
          if (whole) {
            const float inv = lt > 0.f ? 1.f / lt : 0.f;
            const int64_t orow = ((int64_t)b * p.Hq + hk * G + r) * D + half * DW + 4 * q;
#pragma unroll
            for (int mb = 0; mb < MB; ++mb) {
              const f32x4 o = acc[mb] * inv;
              store_out4<QO>(p, orow + 16 * mb, o[0], o[1], o[2], o[3]);
            }
          } else {
            // (own is the same in every lane: the selects stay scalar)
            const bool ow = __builtin_amdgcn_readfirstlane(own ? 1 : 0) != 0;
            float* const cacc = ow ? p.ws_oacc : p.ws_cacc;
            float* const cm = ow ? p.ws_om : p.ws_cm;
            float* const cl = ow ? p.ws_ol : p.ws_cl;
            if (!ow && first_seg && g + nch < g_end) {
              // more segments follow in this share: park the state
#pragma unroll
              for (int mb = 0; mb < MB; ++mb) s_park[half][mb][lane] = acc[mb];
              s_park_ml[half][0][lane] = m;
              s_park_ml[half][1][lane] = lt;
            } else {
              const int64_t row = (ow ? rec * p.rps : (int64_t)slot * p.rps) + r;
              float* ap = cacc + row * D + half * DW + 4 * q;
#pragma unroll
              for (int mb = 0; mb < MB; ++mb) store_state4(ap + 16 * mb, acc[mb], wt);
              if (q == 0 && half == 0) {
                store_state1(cm + row, m, wt);
                store_state1(cl + row, lt, wt);
              }
            }
          }
        }
        if (!whole && !own && first_seg && g + nch < g_end) park_cols = fseg ? nm * G : G;
        if (jA == 0 && lane == 0 && half == 0) {
          // chunks [cs, cs + ncb) of the batch are this stream; the last one
          // lies in the share of wave wave_of(cs + ncb - 1)
          const int last = cs + ncb - 1;
          const int cut = sh_extra * (sh_base + 1);
          const int wl = last < cut ? last / (sh_base + 1) : sh_extra + (last - cut) / sh_base;
          *(int2*)(p.ws_link + 2 * rec) =
              own ? make_int2(-1, 1) : make_int2(slot, whole ? 0 : wl - wx + 1);
        }
      };

      // fold one chunk (its rows in a ring slot, `rows` of them attended)
      auto consume = [&](int rows, const uint4 (&rk)[LPC], const uint4 (&rv)[LPC]) {
        // stage K and V rows in LDS
#pragma unroll
        for (int s = 0; s < LPC; ++s) {
          const int R = s * C::RPI + rowL;
          *(uint4*)(s_k[half] + TR::row(R) + 8 * cc) = rk[s];
          *(uint4*)(s_v[half] + TR::row(R) + 8 * cc) = rv[s];
        }
        // scores of the 16 tokens: lane (q, r) gets tokens 4q..4q+3 of head r
        f32x4 st = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int ks = 0; ks < KS; ++ks) {
          const V8 a = *(const V8*)(s_k[half] + TR::row(r) + 8 * (4 * ks + q));
          if constexpr (kQLds) {
            st = M::mma32(a, s_q[half][0][ks][lane], st);
            st = M::mma32(a, s_q[half][1][ks][lane], st);
          } else {
            st = M::mma32(a, qhi[ks], st);
            st = M::mma32(a, qlo[ks], st);
          }
        }
        if constexpr (DS == 2) {
          // both waves add the two halves in the same order: equal scores
          s_x[par][half][lane] = st;
          __syncthreads();
          st = s_x[par][0][lane] + s_x[par][1][lane];
          par ^= 1;
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
        // 4q + j, columns 16 mb + 4k .. +3 of the V tile (logical chunk
        // 2 mb + k / 2, its half k % 2)
        const int vbase = TR::row(4 * q + tj) + 8 * (tk >> 1) + 4 * (tk & 1);
#pragma unroll
        for (int mb = 0; mb < MB; ++mb) {
          const s16x4 a4 = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
              (lds_s16x4*)(s_v[half] + vbase + 16 * mb));
          const V4 av = __builtin_bit_cast(V4, a4);
          acc[mb] = M::mma16(av, phi, acc[mb]);
          acc[mb] = M::mma16(av, plo, acc[mb]);
        }
      };

      // ---- the ring: slot c % NBUF holds chunk c; chunk c + NBUF - 1 is issued
      // just before chunk c is consumed. The issue is unconditional (a chunk
      // past the end has an empty descriptor and reads nothing), so every path
      // through the loop carries the same loads and the wait before each
      // consume covers only that chunk's loads, not the whole ring.
      uint4 rk[NBUF][LPC], rv[NBUF][LPC];
      int rows[NBUF];
      static_for<0, NBUF - 1>([&](auto S) {
        constexpr int s = decltype(S)::value;
        rows[s] = issue(s, rk[s], rv[s], idr[s]);
      });
      make_q();
      for (int cb = 0; cb < nch; cb += NBUF) {
        static_for<0, NBUF>([&](auto S) {
          constexpr int s = decltype(S)::value;
          constexpr int sn = (s + NBUF - 1) % NBUF;
          const int c = cb + s;
          rows[sn] = issue(c + NBUF - 1, rk[sn], rv[sn], idr[sn]);
          // keep the new chunk's loads ahead of this chunk's wait
          __builtin_amdgcn_sched_barrier(0);
          if (c < nch) {
            consume(rows[s], rk[s], rv[s]);
            if (c + 1 == nch) flush();
          }
        });
      }
    }

    // advance to the next (b, KV head) with chunks
    g += nch;
    j = jA + nch;
    first_seg = false;
    if (j == ncb && g < g_end) {
      j = 0;
      if (++hk == Hkv) {
        hk = 0;
        Pb += ncb;
        do {  // ends: chunks remain, so a non-empty stream follows
          ++v;
          L = F > 0 ? p.ws_vlen[v] : clamped_len(p, v, false);
          ncb = (L + 15) >> 4;
        } while (ncb == 0);
      }
    }
  }
  if (park_cols > 0) {
    // the first segment's state into slot 0, now that no chunk waits follow
    if (r < park_cols) {
      const int64_t row = (int64_t)(2 * wx) * p.rps + r;
      float* ap = p.ws_cacc + row * D + half * DW + 4 * q;
#pragma unroll
      for (int mb = 0; mb < MB; ++mb) store_state4(ap + 16 * mb, s_park[half][mb][lane], wt);
      if (q == 0 && half == 0) {
        store_state1(p.ws_cm + row, s_park_ml[half][0][lane], wt);
        store_state1(p.ws_cl + row, s_park_ml[half][1][lane], wt);
      }
    }
  }
  if (__ballot(bad_block) && lane == 0 && p.status) atomicOr(p.status, kStatusBadBlock);
}

// Ring depth / occupancy / Q' placement / dim split variants per head_dim
// (variant 0 is the default): {NBUF, OCC, Q' in LDS, DS} for head_dim 64, 128,
// 256. At d = 256 one wave holding all dims needs one SIMD to itself; a pair
// splitting them runs at two waves per SIMD like d = 128.
constexpr int kNumVariants = 4;
constexpr int kVariants[kNumVariants][3][4] = {
    {{6, 2, 0, 1}, {3, 2, 0, 1}, {2, 2, 0, 2}},   // 0
    {{12, 1, 0, 1}, {6, 1, 0, 1}, {2, 1, 1, 1}},  // 1
    {{4, 4, 0, 1}, {2, 3, 0, 1}, {3, 2, 1, 2}},   // 2
    {{8, 2, 1, 1}, {4, 2, 1, 1}, {3, 2, 0, 2}},   // 3
};
constexpr int dim_index(int D) { return D == 64 ? 0 : D == 128 ? 1 : 2; }

template <typename T, int D, int V, int POL, int QO>
hipError_t launch_t(const Params& p, hipStream_t s) {
  constexpr int NBUF = kVariants[V][dim_index(D)][0], OCC = kVariants[V][dim_index(D)][1];
  constexpr bool QL = kVariants[V][dim_index(D)][2] != 0;
  constexpr int DS = kVariants[V][dim_index(D)][3];
  // The grid is the host's wave count (waves, or pairs when DS = 2), the same
  // number that sized the workspace's continuation slots: one slot per
  // workgroup of the launch.
  const int workers = p.nwaves;
  if (workers <= 0) return hipErrorInvalidValue;
  hipLaunchKernelGGL((partition_stream_kernel<T, D, NBUF, OCC, POL, QL, QO, DS>), dim3(workers),
                     dim3(64 * DS), 0, s, p);
  return hipGetLastError();
}

// fp32 q/out: every variant; bf16 q/out: the default variant only
template <typename T, int POL>
hipError_t launch_v(const Params& p, int variant, hipStream_t s) {
#define PA_STREAM_CASE(DD)                                          \
  case DD:                                                          \
    if (p.qo_bf16) return launch_t<T, DD, 0, POL, 1>(p, s);         \
    if (variant == 1) return launch_t<T, DD, 1, POL, 0>(p, s);      \
    if (variant == 2) return launch_t<T, DD, 2, POL, 0>(p, s);      \
    if (variant == 3) return launch_t<T, DD, 3, POL, 0>(p, s);      \
    return launch_t<T, DD, 0, POL, 0>(p, s);
  switch (p.D) {
    PA_STREAM_CASE(64)
    PA_STREAM_CASE(128)
    PA_STREAM_CASE(256)
  }
#undef PA_STREAM_CASE
  return hipErrorInvalidValue;
}

template <typename T>
hipError_t launch_d(const Params& p, int variant, bool nt, hipStream_t s) {
  return nt ? launch_v<T, 2>(p, variant, s) : launch_v<T, 0>(p, variant, s);
}

// One wave per group of p.fold consecutive sequences: the folded prefix is the
// run of leading blocks that every member attends whole and whose table
// entries are the same valid block in all members' tables, kept only when it
// is at least kFoldMinTokens long (else 0: every member streams on its own).
// Writes the group's F + 1 virtual lengths: the prefix, then each member's
// clamped length past it (0 for members past the batch).
constexpr int kFoldMinTokens = 256;
__global__ void __launch_bounds__(64) fold_scan_kernel(Params p) {
  const int gi = blockIdx.x, lane = threadIdx.x, F = p.fold;
  const int b0 = gi * F, nm = min(F, p.B - b0);
  // member lane's clamped length (an out-of-range one is reported once)
  const int Lm = lane < nm ? clamped_len(p, b0 + lane, true) : 0x7fffffff;
  int lmin = Lm;
#pragma unroll
  for (int off = 1; off < 64; off <<= 1) lmin = min(lmin, __shfl_xor(lmin, off));
  int pre = 0;
  if (nm >= 2) {
    const int nblk = lmin >> p.bs_log2;  // blocks every member attends whole
    int common = nblk;
    for (int j0 = 0; j0 < nblk; j0 += 64) {
      const int j = j0 + lane;
      bool ok = true;
      if (j < nblk) {
        const int id = p.table[(int64_t)b0 * p.MBS + j];
        ok = id >= 0 && id < p.NB;
        for (int m = 1; m < nm; ++m) ok = ok && p.table[(int64_t)(b0 + m) * p.MBS + j] == id;
      }
      const uint64_t miss = __ballot(!ok);
      if (miss) {
        common = j0 + __builtin_ctzll(miss);
        break;
      }
    }
    pre = common << p.bs_log2;
    if (pre < kFoldMinTokens) pre = 0;
  }
  const int Lprev = __shfl(Lm, (lane + 63) & 63);  // member lane - 1's length
  if (lane <= F) p.ws_vlen[gi * (F + 1) + lane] = lane == 0 ? pre : (lane - 1 < nm ? Lprev - pre : 0);
}

}  // namespace

hipError_t launch_fold_scan(const Params& p, hipStream_t s) {
  if (p.fold <= 0 || p.B <= 0) return hipSuccess;
  const int groups = (p.B + p.fold - 1) / p.fold;
  hipLaunchKernelGGL(fold_scan_kernel, dim3(groups), dim3(64), 0, s, p);
  return hipGetLastError();
}

bool stream_supports(int dtype, int D, int G, int block_size, int batch) {
  return mfma_supports(dtype, D, G) && block_size >= 16 && batch <= kMaxWindows * 64;
}

int stream_grid(int D, int variant, int cus, int64_t chunk_bound) {
  const int v = variant >= 0 && variant < kNumVariants ? variant : 0;
  const int occ = kVariants[v][dim_index(D)][1], ds = kVariants[v][dim_index(D)][3];
  return stream_active_waves(chunk_bound, 4 * occ * cus / ds, cus);
}

hipError_t launch_partition_stream(const Params& p, int dtype, int variant, bool nt, hipStream_t s) {
  if (dtype == 1) return launch_d<_Float16>(p, variant, nt, s);
  if (dtype == 2) return launch_d<__bf16>(p, variant, nt, s);
  return hipErrorInvalidValue;
}

}  // namespace pa
