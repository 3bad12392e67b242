// Prefill-path attention for gfx950 (CDNA4): many new tokens per sequence
// (prompt chunks) over the paged context, one workgroup per (sequence, kv
// head, column block).  The arithmetic is that of the decode kernels in
// attention.hip (QK on the matrix cores, online softmax in fp32, PV on the
// matrix cores), with the context streamed once through LDS for a whole
// block of (new token, query head) columns.

#include "attn_common.h"

namespace pkv {
namespace {

// Compile-time choice between the prefill path's two PV forms (see
// softmax_pv_pair), passed to generic lambdas.
template <bool B>
struct ExactPV {
  static constexpr bool value = B;
};

// Two 16-token sub-tiles at once (16-bit types): QK as two independent MFMA
// chains, one online-softmax update over the 32 tokens, and PV on
// 16x16x32 MFMAs whose K index runs over both sub-tiles.  The K order is a
// fixed permutation of the 32 tokens: lane group r holds k = 8r .. 8r+7,
// taken as tokens 4r .. 4r+3 of the first sub-tile, then of the second.
// That is exactly what each lane holds of P (its QK outputs) and of V (its
// loaded rows), so no operand moves between lanes; A and B only need to
// agree on it.  V comes as the A operands themselves: ve[wd] / vo[wd] hold
// head dim 2 wd / 2 wd + 1 at the lane's four rows of the first sub-tile,
// then its four rows of the second (two bf16/f16 per word).
//
// The softmax reference max is updated lazily: a column keeps its reference
// m while its new logits stay within kLazyLog2 of it (its p stay <= 2^8), and
// the accumulators are rescaled only when some column of the wave moves its
// reference.  o = acc / l holds for any reference, so this changes rounding
// only.  mask (wave-uniform) = false when every real column sees all 32
// tokens; it selects only the logits, so both cases share one instruction
// stream and the accumulators stay in their registers (a separate copy of
// the pair per case made the compiler move all of them at every join).
constexpr float kLazyLog2 = 8.f;

// When a pair may skip the column max.  A pair first weighs its tokens
// against the column's current reference m; only if some lane's weight
// exceeds thr (or is NaN) does it take the column max and apply the lazy
// rule above, then weigh the tokens again.  With a
// finite |m| < 2^22, thr = 16: a column the rule would move has a logit
// above m + 8 up to rounding (above m + 7.5 at that magnitude), whose
// weight is then above 16, so skipping changes nothing.  Without a usable
// reference thr = -1 (always look), except that a padding column (q = 0) with
// none looks once any weight is positive, that is at its first unmasked pair.
struct PairRef {
  float thr;
  __device__ __forceinline__ void set(float m, bool real) {
    thr = __builtin_fabsf(m) < 0x1p22f ? 16.f : (m == kNegInf && !real ? 0.f : -1.f);
  }
};

// QK of a sub-tile pair: two independent MFMA chains.  Issued ahead of the
// softmax of an earlier product, the MFMAs run while the VALU works on it
// (the softmax's rescale branch would otherwise end the scheduling region
// between them).
template <int DT, int N>
__device__ __forceinline__ void qk_pair(const uint4 (&ka0)[N], const uint4 (&ka1)[N],
                                        const uint4 (&qb)[N], floatx4& S0, floatx4& S1) {
  static_assert(DT != DT_F32, "16-bit types only");
  S0 = floatx4{0.f, 0.f, 0.f, 0.f};
  S1 = floatx4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
  for (int kk = 0; kk < N; ++kk) {
    if constexpr (DT == DT_F16) {
      S0 = __builtin_amdgcn_mfma_f32_16x16x32_f16(__builtin_bit_cast(halfx8, ka0[kk]),
                                                  __builtin_bit_cast(halfx8, qb[kk]), S0, 0, 0, 0);
      S1 = __builtin_amdgcn_mfma_f32_16x16x32_f16(__builtin_bit_cast(halfx8, ka1[kk]),
                                                  __builtin_bit_cast(halfx8, qb[kk]), S1, 0, 0, 0);
    } else {
      S0 = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, ka0[kk]),
                                                   __builtin_bit_cast(bf16x8, qb[kk]), S0, 0, 0, 0);
      S1 = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, ka1[kk]),
                                                   __builtin_bit_cast(bf16x8, qb[kk]), S1, 0, 0, 0);
    }
  }
}

// Online softmax and PV of a sub-tile pair whose scores qk_pair produced.
// Two forms of PV:
//  - kExact = false: V arrives as fp16 (bf16 pools are converted when they
//    are parked, exactly for magnitudes in [2^-14, 65504]) and P is rounded
//    to the nearest fp16, one f16 MFMA per product.  P <= 2^8 under the lazy
//    max, so it never overflows; its relative rounding error is at most
//    2^-11, which bounds the error this adds to an output by
//    2^-11 * sum_t p_t |v_t| / l.
//  - kExact = true: V in its storage type and P split into hi + lo 16-bit
//    parts, two MFMAs per product (~16 mantissa bits of P).  Taken where a
//    bf16 V lies outside the fp16 range.
template <int DT, int N, int kMM, bool kExact>
__device__ __forceinline__ void softmax_pv_pair(const floatx4& S0, const floatx4& S1,
                                                const u32x4 (&ve)[N], const u32x4 (&vo)[N],
                                                bool mask, int valid0, int valid1,
                                                float scale_log2, int r, WaveState<kMM>& st,
                                                PairRef& ref, bool real) {
  static_assert(DT != DT_F32, "16-bit types only");
  // Raw scores S; the logit is c * S with c = scale_log2 > 0 (a negative
  // scale arrives as a negated query, a zero one as the smallest normal
  // float).  Multiplying by c > 0 is monotone in floating point, so the
  // largest logit is exactly c * max S, and each exponent is one fma,
  // exp2(c * S - m); a masked score is -inf and gets weight 0.
  float sv[8];
#pragma unroll
  for (int e = 0; e < 4; ++e) {
    sv[e] = S0[e];
    sv[4 + e] = S1[e];
  }
  if (mask) {
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      sv[e] = (4 * r + e < valid0) ? sv[e] : kNegInf;
      sv[4 + e] = (4 * r + e < valid1) ? sv[4 + e] : kNegInf;
    }
  }
  const auto mx = [](float a, float b) { return __builtin_elementwise_maximum(a, b); };
  float pe[8];
  const float nmb = st.m == kNegInf ? 0.f : -st.m;
#pragma unroll
  for (int e = 0; e < 8; ++e) pe[e] = fast_exp2(__builtin_fmaf(sv[e], scale_log2, nmb));
  const float pmax = mx(mx(mx(pe[0], pe[1]), mx(pe[2], pe[3])), mx(mx(pe[4], pe[5]), mx(pe[6], pe[7])));
  if (__builtin_amdgcn_ballot_w64(!(pmax <= ref.thr))) {
    const float mloc =
        scale_log2 * rows_max(mx(mx(mx(sv[0], sv[1]), mx(sv[2], sv[3])), mx(mx(sv[4], sv[5]), mx(sv[6], sv[7]))));
    const bool move = mloc > st.m + kLazyLog2;  // -inf > -inf is false: a fully masked column stays
    if (__builtin_amdgcn_ballot_w64(move)) {
      const float m_new = move ? mloc : st.m;
      const float alpha = move ? fast_exp2(st.m - m_new) : 1.f;
      st.l *= alpha;
#pragma unroll
      for (int mm = 0; mm < kMM; ++mm) st.acc[mm] *= alpha;
      st.m = m_new;
    }
    ref.set(st.m, real);
    const float nmb2 = st.m == kNegInf ? 0.f : -st.m;
#pragma unroll
    for (int e = 0; e < 8; ++e) pe[e] = fast_exp2(__builtin_fmaf(sv[e], scale_log2, nmb2));
  }
  st.l += ((pe[0] + pe[1]) + (pe[2] + pe[3])) + ((pe[4] + pe[5]) + (pe[6] + pe[7]));
  static_assert(kMM == 2 * N, "16-bit types: two head-dim rows per V word");

  if constexpr (!kExact) {
    uint32_t ph[4];
#pragma unroll
    for (int q2 = 0; q2 < 4; ++q2)
      ph[q2] = __builtin_bit_cast(uint32_t,
                                  __builtin_convertvector(floatx2{pe[2 * q2], pe[2 * q2 + 1]}, halfx2));
    const halfx8 P = __builtin_bit_cast(halfx8, make_uint4(ph[0], ph[1], ph[2], ph[3]));
#pragma unroll
    for (int wd = 0; wd < N; ++wd) {  // rows 2 wd and 2 wd + 1 of V^T, fp16
      st.acc[2 * wd] = __builtin_amdgcn_mfma_f32_16x16x32_f16(__builtin_bit_cast(halfx8, ve[wd]), P,
                                                             st.acc[2 * wd], 0, 0, 0);
      st.acc[2 * wd + 1] = __builtin_amdgcn_mfma_f32_16x16x32_f16(__builtin_bit_cast(halfx8, vo[wd]),
                                                                 P, st.acc[2 * wd + 1], 0, 0, 0);
    }
    return;
  }

  uint4 phi, plo;
  uint32_t* ph = reinterpret_cast<uint32_t*>(&phi);
  uint32_t* pl = reinterpret_cast<uint32_t*>(&plo);
#pragma unroll
  for (int q2 = 0; q2 < 4; ++q2) {
    const float p0 = pe[2 * q2], p1 = pe[2 * q2 + 1];
    if constexpr (DT == DT_BF16) {
      const uint32_t b0 = __float_as_uint(p0), b1 = __float_as_uint(p1);
      ph[q2] = __builtin_amdgcn_perm(b1, b0, 0x07060302u);
      const floatx2 lo = {p0 - __uint_as_float(b0 & 0xffff0000u), p1 - __uint_as_float(b1 & 0xffff0000u)};
      pl[q2] = __builtin_bit_cast(uint32_t, __builtin_convertvector(lo, bf16x2));
    } else {
      const fp16x2 hh = __builtin_amdgcn_cvt_pkrtz(p0, p1);
      ph[q2] = __builtin_bit_cast(uint32_t, hh);
      pl[q2] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_pkrtz(p0 - (float)hh[0], p1 - (float)hh[1]));
    }
  }
#pragma unroll
  for (int wd = 0; wd < N; ++wd) {
    const u32x4 ae = ve[wd], ao = vo[wd];  // rows 2 wd and 2 wd + 1 of V^T
    if constexpr (DT == DT_BF16) {
      const bf16x8 hi = __builtin_bit_cast(bf16x8, phi), lo = __builtin_bit_cast(bf16x8, plo);
      const bf16x8 Ae = __builtin_bit_cast(bf16x8, ae), Ao = __builtin_bit_cast(bf16x8, ao);
      st.acc[2 * wd] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(Ae, hi, st.acc[2 * wd], 0, 0, 0);
      st.acc[2 * wd + 1] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(Ao, hi, st.acc[2 * wd + 1], 0, 0, 0);
      st.acc[2 * wd] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(Ae, lo, st.acc[2 * wd], 0, 0, 0);
      st.acc[2 * wd + 1] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(Ao, lo, st.acc[2 * wd + 1], 0, 0, 0);
    } else {
      const halfx8 hi = __builtin_bit_cast(halfx8, phi), lo = __builtin_bit_cast(halfx8, plo);
      const halfx8 Ae = __builtin_bit_cast(halfx8, ae), Ao = __builtin_bit_cast(halfx8, ao);
      st.acc[2 * wd] = __builtin_amdgcn_mfma_f32_16x16x32_f16(Ae, hi, st.acc[2 * wd], 0, 0, 0);
      st.acc[2 * wd + 1] = __builtin_amdgcn_mfma_f32_16x16x32_f16(Ao, hi, st.acc[2 * wd + 1], 0, 0, 0);
      st.acc[2 * wd] = __builtin_amdgcn_mfma_f32_16x16x32_f16(Ae, lo, st.acc[2 * wd], 0, 0, 0);
      st.acc[2 * wd + 1] = __builtin_amdgcn_mfma_f32_16x16x32_f16(Ao, lo, st.acc[2 * wd + 1], 0, 0, 0);
    }
  }
}

// ===========================================================================
// Prefill path: many new tokens per sequence
// ===========================================================================
//
// With L new tokens a sequence has ceil(L * G / 16) column groups; the stream
// kernel streams its context once per group, so a 256-token chunk at G = 4
// reads every K/V byte 64 times.  Here a workgroup takes 4 * GW consecutive
// column groups of one (sequence, kv head), GW per wave, and streams the
// context once for all of them: per stage each wave loads one 16-token
// sub-tile (the block table row read with scalar loads) and parks it in LDS
// (K in the A-operand staging order, V as the PV A operands), and after a
// barrier every wave runs QK, online softmax and PV over the stage's four
// sub-tiles for its own 16 * GW columns, each K/V operand it reads serving
// all of its groups.  The next stage's loads are in flight meanwhile.  A
// workgroup that covers the whole context writes the output rows directly;
// when a call has too few workgroups to fill the chip, each context is cut
// into stage-aligned parts, one workgroup each, and a merge combines the
// parts' states.  Grid: (column block, part) x kv head x sequence rank;
// blocks past a sequence's columns, and empty parts, exit at once.

// kClock: the measurement build, which also records each workgroup that
// streams a context (see clock_record; word 2 adds the sequence, kv head and
// column block, word 3 the part's stages, the part and the context length).
template <int DT, int D, int BS, int GW, bool kClock = false>
__global__ __launch_bounds__(kThreads) __attribute__((amdgpu_waves_per_eu(GW == 2 ? 2 : 3)))
void attn_prefill_kernel(AttnParams prm) {
  [[maybe_unused]] unsigned long long clk0 = 0;
  if constexpr (kClock) clk0 = clock_now();
  static_assert(GW == 1 || (GW == 2 && DT != DT_F32), "two groups per wave: 16-bit types");
  using Geo = Geometry<DT, D, BS>;
  constexpr int N = Geo::N;
  constexpr int kMM = Geo::kMM;
  constexpr int kRow = Geo::kRow;
  constexpr int kSubBytes = kSub * kRow;
  constexpr int kSwz = (4 * N - 1) < 15 ? (4 * N - 1) : 15;
  __shared__ __attribute__((aligned(16))) char sK[1][kWaves][kSubBytes];
  __shared__ __attribute__((aligned(16))) char sV[1][kWaves][kSubBytes];
  __shared__ int sRedo;  // a wave found the fp16 PV form overflowed

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int w = uniform(tid >> 6);
  const int r = lane >> 4;
  if (tid == 0) sRedo = 0;  // read after the stream's barriers
  // Workgroups are dispatched in linear id order, id i to XCD i % 8.  Inside
  // one grid row z (one sequence, kept in its dispatch slot) the ids are
  // dealt so that each (kv head, part) unit goes whole to one XCD, its column
  // blocks one after another: they read the same K/V, which then stays in
  // that XCD's L2.  (Otherwise the ids of the unit's column blocks, being
  // consecutive, landed on every XCD.)
  const int P = prm.prefill_parts;
  const int U = P * (int)gridDim.y;   // units per row
  const int nb = (int)gridDim.x / P;  // column blocks
  const int wrow = (int)blockIdx.x + (int)gridDim.x * (int)blockIdx.y;
  int u, cb;
  if (U % kXcds == 0) {
    const int j = wrow / kXcds;
    u = wrow % kXcds + kXcds * (j / nb);
    cb = j % nb;
  } else {
    u = (int)blockIdx.y * P + (int)blockIdx.x % P;
    cb = (int)blockIdx.x / P;
  }
  const int h = u / P;
  const int part = u % P;
  const int G = prm.group;
  const int Hq = prm.num_q_heads;

  // Longest context first: with up to kPrefillRankSeqs sequences, grid row z
  // takes the sequence whose context is the z-th longest (ties by index), so
  // that the longest workgroups are dispatched first instead of trailing.
  int s = (int)blockIdx.z;
  if (prm.num_seqs <= kPrefillRankSeqs) {
    __shared__ int sN[kPrefillRankSeqs];
    __shared__ int sPick;
    const int B = prm.num_seqs;
    if (tid < B) {
      int c = prm.context_lens[tid];
      sN[tid] = c < 0 ? 0 : (c > prm.max_context_len ? prm.max_context_len : c);
    }
    __syncthreads();
    if (tid < B) {
      const int mine = sN[tid];
      int rank = 0;
      for (int j = 0; j < B; ++j) rank += (sN[j] > mine) || (sN[j] == mine && j < tid);
      if (rank == (int)blockIdx.z) sPick = tid;
    }
    __syncthreads();
    s = uniform(sPick);
  }

  // the sequence's rows, clamped exactly as on the stream path
  int n = prm.context_lens[s];
  n = uniform(n < 0 ? 0 : (n > prm.max_context_len ? prm.max_context_len : n));
  const int T = prm.num_query_tokens;
  int q0 = prm.query_start[s], qe = prm.query_start[s + 1];
  q0 = q0 < 0 ? 0 : (q0 > T ? T : q0);
  qe = qe < q0 ? q0 : (qe > T ? T : qe);
  int L = qe - q0;
  L = L < n ? L : n;
  L = L < prm.max_query_len ? L : prm.max_query_len;
  q0 = uniform(q0);
  L = uniform(L);
  const int ngrp = (L * G + kSub - 1) / kSub;
  // column groups per wave (kGW) and per workgroup (kGB)
  constexpr int kGW = GW;
  constexpr int kGB = kWaves * kGW;
  if (cb * kGB >= ngrp) return;  // the whole workgroup: no barrier follows

  SeqCols sc;
  sc.n = n;
  sc.L = L;
  sc.q0 = q0;
  sc.ngrp = ngrp;
  const int cg0 = cb * kGB + w * kGW;  // this wave's first group
  uint4 qb[kGW][N];
#pragma unroll
  for (int g = 0; g < kGW; ++g) load_query_cols<N, true>(qb[g], prm.q, sc, h, cg0 + g, G, Hq, lane);
  // 16-bit types: the core takes a non-negative logit scale; a negative one
  // becomes a negated query (a sign flip, exact)
  const bool neg_scale = prm.scale_log2 < 0.f;
  if constexpr (DT != DT_F32)
    if (neg_scale)
#pragma unroll
      for (int g = 0; g < kGW; ++g)
#pragma unroll
        for (int kk = 0; kk < N; ++kk) {
          qb[g][kk].x ^= 0x80008000u;
          qb[g][kk].y ^= 0x80008000u;
          qb[g][kk].z ^= 0x80008000u;
          qb[g][kk].w ^= 0x80008000u;
        }
  // per group: tokens this lane's column sees, and tokens every real column
  // of the group sees (its first column's); 0 for a group past the last
  int vis[kGW], vis_first[kGW];
#pragma unroll
  for (int g = 0; g < kGW; ++g) {
    const int col = (cg0 + g) * kSub + (lane & 15);
    vis[g] = col < L * G ? n - L + col / G + 1 : 0;
    vis_first[g] = cg0 + g < ngrp ? n - L + ((cg0 + g) * kSub) / G + 1 : 0;
  }
  // tokens the last column of this wave's groups / of the block's last group sees
  auto group_limit = [&](int g) {
    int i_last = (g * kSub + kSub - 1) / G;
    i_last = i_last < L - 1 ? i_last : L - 1;
    return n - L + i_last + 1;
  };
  const int cg_w = cg0 + kGW - 1 < ngrp ? cg0 + kGW - 1 : ngrp - 1;
  const int nsub_w = cg0 < ngrp ? (group_limit(cg_w) + kSub - 1) / kSub : 0;
  const int cg_last = (cb + 1) * kGB < ngrp ? (cb + 1) * kGB - 1 : ngrp - 1;
  const int rows_b = group_limit(cg_last);
  const int nsub_b = (rows_b + kSub - 1) / kSub;
  const int nstage_all = (nsub_b + kWaves - 1) / kWaves;
  // this workgroup's part of the context: stages [st0, st1)
  const int per_part = (nstage_all + P - 1) / P;
  const int st0 = part * per_part;
  const int st1 = st0 + per_part < nstage_all ? st0 + per_part : nstage_all;
  if (st0 >= st1) return;  // an empty part: the merge skips it
  const int sub_end = st1 * kWaves < nsub_b ? st1 * kWaves : nsub_b;

  typedef const __attribute__((address_space(4))) int32_t const_i32;
  const_i32* row_ids = (const_i32*)prm.block_tables + (size_t)s * prm.max_blocks_per_seq;
  const int koff = 16 * lane;
  const int voff = (4 * r) * kRow + (lane & 15) * (4 * N);

  // Sub-tile `sub` of the context into t; past the block's last visible row
  // (or for an id outside the pool) the rows read as zeros, touching nothing.
  auto load_sub = [&](Tile<N>& t, int sub) {
    const char* kb = static_cast<const char*>(prm.k_cache);
    const char* vb = static_cast<const char*>(prm.v_cache);
    int nrec = 0;
    if (sub < sub_end) {
      const int blk = sub * kSub / BS;  // < ceil(rows_b / BS) <= max_blocks_per_seq
      int phys = row_ids[blk];
      const bool ok = (unsigned)phys < (unsigned)prm.num_blocks;
      phys = ok ? phys : 0;
      int rows = rows_b - sub * kSub;
      rows = rows > kSub ? kSub : rows;
      const size_t off = ((size_t)phys * prm.num_kv_heads + h) * Geo::kTileBytes +
                         (sub * kSub % BS) * kRow;
      nrec = uniform(ok ? rows * kRow : 0);
      kb += off;
      vb += off;
    }
    load_tile<N>(t, make_rsrc(kb, nrec), make_rsrc(vb, nrec), koff, voff);
  };
  // This wave's loaded sub-tile into slot w of stage buffer b: K chunk c of
  // token row t at chunk position c ^ (t & mask) (as restage_k stores it),
  // V as the lanes hold it (bf16 V converted to fp16 for the fp16 PV form).
  auto park = [&](const Tile<N>& t, int b, auto exact) {
    constexpr bool kEx = decltype(exact)::value;
#pragma unroll
    for (int kk = 0; kk < N; ++kk) {
      const int o = 1024 * kk + 16 * lane;
      const int tr = o / kRow, c = (o % kRow) / 16;
      *reinterpret_cast<uint4*>(&sK[b][w][tr * kRow + ((c ^ (tr & kSwz)) * 16)]) = t.k[kk];
    }
#pragma unroll
    for (int qd = 0; qd < N; ++qd) {
      if constexpr (DT == DT_F32) {
        *reinterpret_cast<uint4*>(&sV[b][w][(qd * 64 + lane) * 16]) =
            make_uint4(t.v[0][qd], t.v[1][qd], t.v[2][qd], t.v[3][qd]);
      } else {
        // The PV A-operand words of dim pair qd: even dim at rows 0-1, 2-3,
        // odd dim likewise.  Sub-tiles 2p and 2p + 1 of a stage form pair p,
        // whose two slots hold, per (qd, even/odd, lane), the first
        // sub-tile's two words then the second's: attend_pair reads each
        // operand with one load.
        uint2 ev, od;
        if constexpr (DT == DT_BF16 && !kEx) {
          // bf16 -> fp32 is a shift of the bits; fp32 -> fp16 rounds to
          // nearest (exact for every bf16 in the fp16 range; above it, +-inf)
          auto f16x2 = [](uint32_t lo_bits, uint32_t hi_bits) {
            return __builtin_bit_cast(
                uint32_t, __builtin_convertvector(
                              floatx2{__uint_as_float(lo_bits), __uint_as_float(hi_bits)}, halfx2));
          };
          ev.x = f16x2(t.v[0][qd] << 16, t.v[1][qd] << 16);
          ev.y = f16x2(t.v[2][qd] << 16, t.v[3][qd] << 16);
          od.x = f16x2(t.v[0][qd] & 0xffff0000u, t.v[1][qd] & 0xffff0000u);
          od.y = f16x2(t.v[2][qd] & 0xffff0000u, t.v[3][qd] & 0xffff0000u);
        } else {
          ev.x = __builtin_amdgcn_perm(t.v[1][qd], t.v[0][qd], 0x05040100u);
          ev.y = __builtin_amdgcn_perm(t.v[3][qd], t.v[2][qd], 0x05040100u);
          od.x = __builtin_amdgcn_perm(t.v[1][qd], t.v[0][qd], 0x07060302u);
          od.y = __builtin_amdgcn_perm(t.v[3][qd], t.v[2][qd], 0x07060302u);
        }
        char* pair = &sV[b][w & ~1][0] + 8 * (w & 1);
        *reinterpret_cast<uint2*>(pair + ((2 * qd) * 64 + lane) * 16) = ev;
        *reinterpret_cast<uint2*>(pair + ((2 * qd + 1) * 64 + lane) * 16) = od;
      }
    }
  };

  WaveState<kMM> st[kGW];
  PairRef ref[kGW];
  // fp32 scales its logits directly.  16-bit types take |scale| (see above),
  // and a zero scale as the smallest normal float: every logit c * S is then
  // within 2^-24 of zero for |S| < 2^100, so every weight exp2(c * S - m)
  // rounds to exactly 1 as it would for c = 0, while a masked -inf stays -inf.
  float scale_log2 = DT != DT_F32 && neg_scale ? -prm.scale_log2 : prm.scale_log2;
  if constexpr (DT != DT_F32)
    if (scale_log2 == 0.f) scale_log2 = 1.17549435e-38f;
  // QK, softmax and PV over the four sub-tiles of stage sg (LDS buffer b).
  auto fetch_k = [&](uint4 (&ka)[N], int b, int j) {
    const int tr = lane & 15;
#pragma unroll
    for (int kk = 0; kk < N; ++kk) {
      const int c = (lane >> 4) + 4 * kk;
      ka[kk] = *reinterpret_cast<const uint4*>(&sK[b][j][tr * kRow + ((c ^ (tr & kSwz)) * 16)]);
    }
  };
  auto fetch_v = [&](u32x4 (&va)[N], int b, int j) {
#pragma unroll
    for (int qd = 0; qd < N; ++qd) va[qd] = *reinterpret_cast<const u32x4*>(&sV[b][j][(qd * 64 + lane) * 16]);
  };
  // V operands of pair p (sub-tiles 2p, 2p + 1), as park lays them out
  auto fetch_v_pair = [&](u32x4 (&ve)[N], u32x4 (&vo)[N], int b, int p) {
    const char* pair = &sV[b][2 * p][0];
#pragma unroll
    for (int qd = 0; qd < N; ++qd) {
      ve[qd] = *reinterpret_cast<const u32x4*>(pair + ((2 * qd) * 64 + lane) * 16);
      vo[qd] = *reinterpret_cast<const u32x4*>(pair + ((2 * qd + 1) * 64 + lane) * 16);
    }
  };
  auto valid_of = [&](int g, int sub) {
    const int v = vis[g] - sub * kSub;
    return v > kSub ? kSub : v;
  };
  // QK, softmax and PV over the four sub-tiles of stage sg (LDS buffer b):
  // two pairs for 16-bit types, each pair's K and V operands read once and
  // used by both of the wave's groups (a pair whose second sub-tile is past
  // a group's limit masks it: every token there is past every column's
  // limit), four single sub-tiles for fp32.
  auto compute_stage = [&](int sg, int b, auto exact) {
    constexpr bool kEx = decltype(exact)::value;
    if constexpr (DT != DT_F32) {
#pragma unroll
      for (int j = 0; j < kWaves; j += 2) {
        const int sub = sg * kWaves + j;
        if (sub < nsub_w) {
          uint4 ka0[N], ka1[N];
          u32x4 ve[N], vo[N];
          fetch_k(ka0, b, j);
          fetch_k(ka1, b, j + 1);
          // every group's QK first, then each group's softmax and PV
          floatx4 S[kGW][2];
#pragma unroll
          for (int g = 0; g < kGW; ++g) qk_pair<DT, N>(ka0, ka1, qb[g], S[g][0], S[g][1]);
          fetch_v_pair(ve, vo, b, j / 2);
#pragma unroll
          for (int g = 0; g < kGW; ++g) {
            const bool mask = (sub + 2) * kSub > vis_first[g];
            softmax_pv_pair<DT, N, kMM, kEx>(S[g][0], S[g][1], ve, vo, mask, valid_of(g, sub),
                                             valid_of(g, sub + 1), scale_log2, r, st[g], ref[g],
                                             vis[g] > 0);
          }
        }
      }
    } else {
#pragma unroll
      for (int j = 0; j < kWaves; ++j) {
        const int sub = sg * kWaves + j;
        if (sub < nsub_w) {
          uint4 ka[N];
          u32x4 va[N];
          uint32_t vv[4][N];
          fetch_k(ka, b, j);
          fetch_v(va, b, j);
#pragma unroll
          for (int qd = 0; qd < N; ++qd) {
            vv[0][qd] = va[qd].x;
            vv[1][qd] = va[qd].y;
            vv[2][qd] = va[qd].z;
            vv[3][qd] = va[qd].w;
          }
          attend_core<DT, N, kMM>(ka, vv, qb[0], valid_of(0, sub), scale_log2, r, st[0]);
        }
      }
    }
  };
  // One register tile keeps this wave's sub-tile of the next stage in flight
  // while the current stage is computed from LDS; it is parked in the other
  // buffer (whose last readers finished before the previous barrier).  (A
  // ring of three tiles measured no faster: the core, not the loads, sets
  // the pace.)
  auto stream_context = [&](auto exact) {
#pragma unroll
    for (int g = 0; g < kGW; ++g) {
      st[g].reset();
      ref[g].set(kNegInf, vis[g] > 0);
    }
    Tile<N> t;
    load_sub(t, st0 * kWaves + w);
    park(t, 0, exact);
    __syncthreads();
    for (int sg = st0; sg < st1; ++sg) {
      // With the contexts cut into parts every workgroup has the same work,
      // and those sharing a compute unit otherwise progress at the issue
      // arbiter's whim (the older waves first), the last then running alone;
      // the waves with more of their part left go first, so that they keep
      // pace.  (Uncut contexts differ in length and are dispatched longest
      // first: there it made no difference or cost a little.)
      if (P > 1) {
        const int left = st1 - sg;
        if (left > 48)
          __builtin_amdgcn_s_setprio(3);
        else if (left > 24)
          __builtin_amdgcn_s_setprio(2);
        else if (left > 8)
          __builtin_amdgcn_s_setprio(1);
        else
          __builtin_amdgcn_s_setprio(0);
      }
      load_sub(t, (sg + 1) * kWaves + w);
      compute_stage(sg, 0, exact);
      __syncthreads();  // every wave has read the stage
      park(t, 0, exact);
      __syncthreads();
    }
  };
  // 16-bit types take the fp16 PV form.  A bf16 V element beyond the fp16
  // range became +-inf there, which leaves some accumulator of the
  // workgroup non-finite (inf * p, or 0 * inf = NaN where p = 0), so the
  // workgroup then streams its context again in the exact form (as it does,
  // at no harm but the time, for non-finite inputs).
  stream_context(ExactPV<DT == DT_F32>{});
  if constexpr (DT == DT_BF16) {
    float sum = 0.f;
#pragma unroll
    for (int g = 0; g < kGW; ++g)
#pragma unroll
      for (int mm = 0; mm < kMM; ++mm) sum += (st[g].acc[mm][0] + st[g].acc[mm][1]) + (st[g].acc[mm][2] + st[g].acc[mm][3]);
    const bool bad = !(sum - sum == 0.f);  // inf - inf and NaN - NaN are NaN
    if (__builtin_amdgcn_ballot_w64(bad) != 0 && lane == 0) sRedo = 1;
    __syncthreads();
    if (sRedo) stream_context(ExactPV<true>{});
  }


  if constexpr (kClock)
    if (tid == 0)
      clock_record(prm.clock,
                   (long long)blockIdx.x + (long long)gridDim.x * (blockIdx.y + (long long)gridDim.y * blockIdx.z),
                   clk0, (unsigned long long)s | ((unsigned long long)h << 24) | ((unsigned long long)cb << 40),
                   (unsigned long long)(st1 - st0) | ((unsigned long long)part << 20) |
                       ((unsigned long long)n << 32));
#pragma unroll
  for (int g = 0; g < kGW; ++g) {
    if (cg0 + g >= ngrp) break;
    float l = st[g].l + __shfl_xor(st[g].l, 16);
    l += __shfl_xor(l, 32);
    float o[D / 4];
    lane_run<D, kMM>(o, st[g]);
    const int col = (cg0 + g) * kSub + (lane & 15);
    if (col < L * G) {
      const size_t orow = (size_t)(q0 + col / G) * Hq + (size_t)h * G + col % G;
      if (P == 1) {
        const float inv = l > 0.f ? 1.f / l : 0.f;
#pragma unroll
        for (int i = 0; i < D / 4; ++i) o[i] *= inv;
        store_run<DT, D>(static_cast<char*>(prm.out) + (orow * D + r * (D / 4)) * Geo::EB, o);
      } else {
        // part state: unnormalised o, running max (log2 units), normaliser
        const size_t slot = orow * P + part;
        store_run<DT_F32, D>(prm.part_o + slot * D + r * (D / 4), o);
        if (r == 0) *reinterpret_cast<float2*>(prm.part_ml + slot * 2) = make_float2(st[g].m, l);
      }
    }
  }
}

// New tokens of sequence s with a context of n tokens, clamped as every
// kernel clamps them: [query_start[s], query_start[s+1]) inside [0, rows],
// at most min(n, max_query_len).
__device__ __forceinline__ int clamped_new_tokens(const AttnParams& prm, int s, int n, int* q0_out) {
  const int T = prm.num_query_tokens;
  int q0 = prm.query_start[s], qe = prm.query_start[s + 1];
  q0 = q0 < 0 ? 0 : (q0 > T ? T : q0);
  qe = qe < q0 ? q0 : (qe > T ? T : qe);
  int L = qe - q0;
  L = L < n ? L : n;
  L = L < prm.max_query_len ? L : prm.max_query_len;
  if (q0_out) *q0_out = q0;
  return L;
}

// Merge of split prefill contexts: eight (query row, query head) items per
// wave, eight lanes per item, each lane D / 8 of the head dim, parts in
// order: each lane sums its values over the parts exactly as a whole wave
// per item did, with eight times fewer waves.  Items past a sequence's rows
// exit at once.  The number of non-empty parts follows from the same stage
// counts the prefill kernel uses.  Grid: one thread per (item, lane).
constexpr int kMergeLanes = 8;

template <int DT, int NV>
__device__ __forceinline__ void store_vals(void* dst, const float (&o)[NV]) {
  if constexpr (DT == DT_F32) {
#pragma unroll
    for (int i = 0; i < NV / 4; ++i)
      reinterpret_cast<float4*>(dst)[i] = make_float4(o[4 * i], o[4 * i + 1], o[4 * i + 2], o[4 * i + 3]);
  } else {
    uint32_t packed[NV / 2];
#pragma unroll
    for (int i = 0; i < NV / 2; ++i) {
      uint16_t lo, hi;
      if constexpr (DT == DT_F16) {
        lo = __builtin_bit_cast(uint16_t, (_Float16)o[2 * i]);
        hi = __builtin_bit_cast(uint16_t, (_Float16)o[2 * i + 1]);
      } else {
        lo = f32_to_bf16_rne(o[2 * i]);
        hi = f32_to_bf16_rne(o[2 * i + 1]);
      }
      packed[i] = (uint32_t)lo | ((uint32_t)hi << 16);
    }
#pragma unroll
    for (int i = 0; i < NV / 8; ++i)
      reinterpret_cast<uint4*>(dst)[i] =
          make_uint4(packed[4 * i], packed[4 * i + 1], packed[4 * i + 2], packed[4 * i + 3]);
  }
}

template <int DT, int D>
__global__ __launch_bounds__(kThreads) void attn_prefill_merge_kernel(AttnParams prm) {
  constexpr int kF = D / kMergeLanes;  // head-dim values per lane
  const long long item = ((long long)blockIdx.x * kThreads + threadIdx.x) / kMergeLanes;
  const int sub = (int)(threadIdx.x % kMergeLanes);
  const int Hq = prm.num_q_heads;
  const int G = prm.group;
  const int P = prm.prefill_parts;
  const int hq = (int)(item % Hq);
  const long long rest = item / Hq;
  const int i = (int)(rest % prm.max_query_len);
  const long long sl = rest / prm.max_query_len;
  if (sl >= prm.num_seqs) return;
  const int s = (int)sl;
  int n = prm.context_lens[s];
  n = n < 0 ? 0 : (n > prm.max_context_len ? prm.max_context_len : n);
  int q0;
  const int L = clamped_new_tokens(prm, s, n, &q0);
  if (i >= L) return;
  const int Ps = P;
  const int kGB = kWaves * prm.prefill_wave_groups;  // groups per column block
  const int c = i * G + hq % G;  // the column, in its kv head's block
  const int cb = c / (kGB * kSub);
  const int ngrp = (L * G + kSub - 1) / kSub;
  const int cg_last = (cb + 1) * kGB < ngrp ? (cb + 1) * kGB - 1 : ngrp - 1;
  int i_last = (cg_last * kSub + kSub - 1) / G;
  i_last = i_last < L - 1 ? i_last : L - 1;
  const int rows_b = n - L + i_last + 1;
  const int nstage_all = ((rows_b + kSub - 1) / kSub + kWaves - 1) / kWaves;
  const int per_part = (nstage_all + Ps - 1) / Ps;
  const int nparts = (nstage_all + per_part - 1) / per_part;
  const size_t base = ((size_t)(q0 + i) * Hq + hq) * P;

  float M = kNegInf;
  for (int k = 0; k < nparts; ++k) M = fmaxf(M, prm.part_ml[(base + k) * 2]);
  float o[kF];
#pragma unroll
  for (int j = 0; j < kF; ++j) o[j] = 0.f;
  float lsum = 0.f;
  for (int k = 0; k < nparts; ++k) {
    const float2 ml = *reinterpret_cast<const float2*>(prm.part_ml + (base + k) * 2);
    const float f = ml.x == kNegInf ? 0.f : fast_exp2(ml.x - M);
    lsum += f * ml.y;
    const float4* src = reinterpret_cast<const float4*>(prm.part_o + (base + k) * D + sub * kF);
#pragma unroll
    for (int j = 0; j < kF / 4; ++j) {
      const float4 x = src[j];
      o[4 * j] += f * x.x;
      o[4 * j + 1] += f * x.y;
      o[4 * j + 2] += f * x.z;
      o[4 * j + 3] += f * x.w;
    }
  }
  const float inv = lsum > 0.f ? 1.f / lsum : 0.f;
#pragma unroll
  for (int j = 0; j < kF; ++j) o[j] *= inv;
  const size_t orow = ((size_t)(q0 + i) * Hq + hq) * D + (size_t)sub * kF;
  store_vals<DT, kF>(static_cast<char*>(prm.out) + orow * Elem<DT>::bytes, o);
}

template <int DT, int D, int BS>
hipError_t launch_prefill_typed(const AttnParams& prm, hipStream_t stream) {
  const dim3 block(kThreads);
  const long long nout = (long long)prm.num_seqs * prm.num_q_heads;
  if (nout > 0x7fffffffLL) return hipErrorInvalidConfiguration;
  {
    const long long nx = (long long)prm.prefill_blocks * prm.prefill_parts;
    if (!prm.query_start || prm.num_seqs > 65535 || prm.num_kv_heads > 65535 ||
        prm.prefill_parts < 1 || nx > 0x7fffffffLL)
      return hipErrorInvalidConfiguration;
    const dim3 grid((unsigned)nx, (unsigned)prm.num_kv_heads, (unsigned)prm.num_seqs);
    // the clock build: a measurement variant of one shape (bf16, D 128,
    // 16-token blocks)
    constexpr bool kClockBuilt = DT == DT_BF16 && D == 128 && BS == 16;
    const bool clock = prm.clock != nullptr && kClockBuilt;
    if (prm.prefill_wave_groups == 1) {
      if (clock)
        hipLaunchKernelGGL((attn_prefill_kernel<DT, D, BS, 1, kClockBuilt>), grid, block, 0, stream, prm);
      else
        hipLaunchKernelGGL((attn_prefill_kernel<DT, D, BS, 1>), grid, block, 0, stream, prm);
    } else if constexpr (DT != DT_F32) {
      if (clock)
        hipLaunchKernelGGL((attn_prefill_kernel<DT, D, BS, 2, kClockBuilt>), grid, block, 0, stream, prm);
      else
        hipLaunchKernelGGL((attn_prefill_kernel<DT, D, BS, 2>), grid, block, 0, stream, prm);
    } else {
      return hipErrorInvalidValue;
    }
    hipError_t err = hipGetLastError();
    if (err != hipSuccess || prm.prefill_parts == 1) return err;
    const long long threads =
        (long long)prm.num_seqs * prm.max_query_len * prm.num_q_heads * kMergeLanes;
    const long long nm = (threads + kThreads - 1) / kThreads;
    if (nm > 0x7fffffffLL) return hipErrorInvalidConfiguration;
    hipLaunchKernelGGL((attn_prefill_merge_kernel<DT, D>), dim3((unsigned)nm), block, 0, stream,
                       prm);
    return hipGetLastError();
  }
}

template <int DT, int D>
hipError_t launch_prefill_bs(const AttnParams& prm, int bs, hipStream_t stream) {
  switch (bs) {
    case 16: return launch_prefill_typed<DT, D, 16>(prm, stream);
    case 32: return launch_prefill_typed<DT, D, 32>(prm, stream);
    default: return hipErrorInvalidValue;
  }
}

template <int DT>
hipError_t launch_prefill_d(const AttnParams& prm, int d, int bs, hipStream_t stream) {
  switch (d) {
    case 64: return launch_prefill_bs<DT, 64>(prm, bs, stream);
    case 128: return launch_prefill_bs<DT, 128>(prm, bs, stream);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace

int32_t prefill_parts_for(int32_t num_seqs, int32_t num_kv_heads, int32_t prefill_blocks,
                          int32_t max_context_len) {
  const long long wgs = (long long)num_seqs * num_kv_heads * prefill_blocks;
  if (wgs <= 0 || wgs >= kPrefillMinWorkgroups) return 1;
  long long p = (kPrefillMinWorkgroups + wgs - 1) / wgs;
  const long long by_len = max_context_len / kPrefillMinPartTokens;
  if (p > by_len) p = by_len;
  if (p > kPrefillMaxParts) p = kPrefillMaxParts;
  return p < 1 ? 1 : (int32_t)p;
}

PrefillPlan prefill_plan(int32_t num_seqs, int32_t num_kv_heads, int32_t max_groups,
                         int32_t max_context_len, int dtype) {
  auto blocks_of = [&](int32_t gw) { return (max_groups + kWaves * gw - 1) / (kWaves * gw); };
  PrefillPlan pl{1, blocks_of(1), 1};
  if (dtype != DT_F32) {
    const long long wgs2 = (long long)num_seqs * num_kv_heads * blocks_of(2);
    if (wgs2 < kPrefillMinWorkgroups || wgs2 >= 2LL * kPrefillMinWorkgroups)
      pl = PrefillPlan{2, blocks_of(2), 1};
  }
  pl.parts = prefill_parts_for(num_seqs, num_kv_heads, pl.blocks, max_context_len);
  return pl;
}

AttnWorkspace prefill_workspace_layout(int32_t num_query_tokens, int32_t num_q_heads,
                                       int32_t head_dim, int32_t parts) {
  AttnWorkspace ws{0, 0, 0, 0};
  if (parts <= 1 || num_query_tokens <= 0 || num_q_heads <= 0 || head_dim <= 0) return ws;
  const size_t slots = (size_t)num_query_tokens * num_q_heads * parts;
  ws.part_o_off = 0;
  ws.part_ml_off = align256(slots * head_dim * sizeof(float));
  ws.bytes = ws.part_ml_off + slots * 2 * sizeof(float);
  return ws;
}

hipError_t launch_prefill(const AttnParams& prm, int dtype, int head_dim, int block_size,
                          hipStream_t stream) {
  switch (dtype) {
    case DT_F32: return launch_prefill_d<DT_F32>(prm, head_dim, block_size, stream);
    case DT_F16: return launch_prefill_d<DT_F16>(prm, head_dim, block_size, stream);
    case DT_BF16: return launch_prefill_d<DT_BF16>(prm, head_dim, block_size, stream);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace pkv
