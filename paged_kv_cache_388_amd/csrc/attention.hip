// Paged decode attention for gfx950 (CDNA4).
//
// What is computed: for each sequence s and query head h, attention of the
// single new query over the sequence's cached context, gathered through its
// block table (first page, "PagedAttention: Decoupling Logical Context from
// Contiguous GPU Memory"; "The Memory Wall", "Show Me The Code: A Conceptual
// PagedAttention Kernel", whose loop over logical blocks with one table lookup
// per block is the structure kept here).  Query head h reads KV head h / G.
//
// The unit of work is a 16-token sub-tile of one (kv head, sequence): all G
// query heads of the kv head share the K/V bytes it streams, so every K/V byte
// crosses HBM once per call.  Per sub-tile a wave does:
//   QK   S^T[16 tok x 16 cols] = K_tile[16 x D] . Q^T[D x 16] on MFMA
//        (16x16x32 for fp16/bf16, 16x16x4 for fp32).  Column g < G is query
//        head h*G+g; the other columns are zero padding.  K is loaded as whole
//        128-byte lines and re-dealt into the MFMA operand layout through the
//        wave's LDS slot.
//   mask tokens at or past the context length get -inf (a select, so stale
//        or NaN bits in unused slots never reach the result).
//   softmax  running max per column (3 ops in-lane + 2 cross-row shuffles),
//        exp2 of base-2 logits, running normaliser, rescale of the
//        accumulator when the max grows.
//   PV   O^T[D x 16] += V^T[D x 16 tok] . P^T[16 tok x 16] on MFMA
//        (16x16x16).  P^T is the QK result already in place.  V^T is built
//        from natural V loads: the head-dim index d is permuted so that MFMA
//        row rho, pass mm holds d = (D/16)*rho + mm, which makes each lane's
//        four token chunks the four k-values of its A operand (one v_perm_b32
//        per pair).  P is split into hi + lo 16-bit parts so the product keeps
//        ~16 mantissa bits instead of 8.
//
// Stream path (batches up to kMaxStreamSeqs).  The work of a call is the
// ordered list of positions (kv head, sequence, sub-tile).  Two workgroups per
// CU stay resident for the whole call; each of their waves owns one equal,
// contiguous chunk of that list and streams it through a 3-deep register ring
// that runs across sequence boundaries, so every wave has the same number of
// tiles and no slot idles between items.  The blockIdx -> chunk map is
// XCD-aware: each XCD takes one contiguous range of the list (one kv head at
// H_kv = 8), so sequences sharing blocks meet in the same L2.  A wave writes a
// sequence it covers whole straight to `out`; a piece of a longer sequence
// goes to one of the wave's two partial slots (its first and last piece), and
// a second kernel merges the pieces of each split sequence in logical order.
//
// Grid path (larger batches).  One workgroup of 4 waves per (kv head,
// sequence, 512-token partition); wave w takes sub-tiles w, w+4, ...; the
// waves merge in LDS and a second kernel merges the partitions.
//
// In both, every reduction order depends only on logical token positions and
// context lengths, never on physical block ids or on which workgroup ran
// what, so the result is bit-identical under any physical placement.


#include <hip/hip_runtime.h>
#include <stdint.h>

#include "kernels.h"

namespace pkv {
namespace {

typedef float floatx4 __attribute__((ext_vector_type(4)));
typedef float floatx2 __attribute__((ext_vector_type(2)));
typedef short shortx4 __attribute__((ext_vector_type(4)));
typedef _Float16 halfx4 __attribute__((ext_vector_type(4)));
typedef _Float16 halfx8 __attribute__((ext_vector_type(8)));
typedef __fp16 fp16x2 __attribute__((ext_vector_type(2)));  // cvt_pkrtz result
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef _Float16 halfx2 __attribute__((ext_vector_type(2)));
typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));

// Compile-time choice between the prefill path's two PV forms (see
// softmax_pv_pair), passed to generic lambdas.
template <bool B>
struct ExactPV {
  static constexpr bool value = B;
};

constexpr int kWaves = kStreamWaves;  // waves per workgroup, both paths
constexpr int kThreads = 64 * kWaves;
constexpr int kSub = kSubTokens;      // tokens per MFMA row group
constexpr int kXcds = 8;
constexpr float kNegInf = -__builtin_huge_valf();

enum { DT_F32 = 0, DT_F16 = 1, DT_BF16 = 2 };

template <int DT> struct Elem { static constexpr int bytes = 2; };
template <> struct Elem<DT_F32> { static constexpr int bytes = 4; };

// Workgroups are dispatched round-robin over the 8 XCDs.  Remap the linear id
// so each XCD receives one contiguous range of the logical work order (kv
// head slowest): the sequences that read the same kv head's blocks, shared
// prefixes included, then meet in the same L2.
__device__ __forceinline__ int xcd_remap(int bid, int nblocks) {
  const int per = nblocks / kXcds, rem = nblocks % kXcds;
  const int xcd = bid % kXcds, local = bid / kXcds;
  const int start = xcd < rem ? xcd * (per + 1) : rem * (per + 1) + (xcd - rem) * per;
  return start + local;
}

__device__ __forceinline__ uint16_t f32_to_bf16_rne(float f) {
  uint32_t u = __float_as_uint(f);
  if ((u & 0x7fffffffu) > 0x7f800000u) return (uint16_t)((u >> 16) | 0x40u);
  u += 0x7fffu + ((u >> 16) & 1u);
  return (uint16_t)(u >> 16);
}

template <int DT>
__device__ __forceinline__ void store_out(void* out, size_t idx, float v) {
  if constexpr (DT == DT_F32) {
    static_cast<float*>(out)[idx] = v;
  } else if constexpr (DT == DT_F16) {
    static_cast<_Float16*>(out)[idx] = (_Float16)v;
  } else {
    static_cast<uint16_t*>(out)[idx] = f32_to_bf16_rne(v);
  }
}

__device__ __forceinline__ float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }

__device__ __forceinline__ int uniform(int x) { return __builtin_amdgcn_readfirstlane(x); }

// Raw buffer resource over one (block, head) tile: the base is uniform
// (scalar registers), so a tile costs a few scalar ops plus two per-lane
// offsets that never change.  Offsets at or past num_records read as zero
// without touching memory.
typedef __amdgpu_buffer_rsrc_t rsrc_t;
constexpr int kRsrcWord3 = 0x00020000;  // raw 32-bit-dword buffer, gfx9 family
// K and V bytes are read once per step: load them with the nontemporal cache
// policy ("nt") so they stream through the caches instead of displacing
// lines, which lifts sustained read bandwidth substantially on gfx950.
constexpr int kStreamPolicy = 2;

__device__ __forceinline__ rsrc_t make_rsrc(const void* base, int num_bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0, num_bytes, kRsrcWord3);
}

// One 16-token sub-tile in registers.  N = D * elem_bytes / 64.
//   k[kk]   : bytes [1024*kk + 16*lane, +16) of the sub-tile (each load
//             instruction reads 1 KiB of whole token rows)
//   v[e][.] : token 4*(lane >> 4) + e, bytes [(lane & 15)*4N, +4N) of its row
// Both patterns cover whole 128-byte lines per instruction, which the
// nontemporal loads need to stream at full rate; a pattern that touches half
// lines (16 rows x 64 bytes, the MFMA operand layout) runs ~15% slower.
template <int N>
struct Tile {
  uint4 k[N];
  uint32_t v[4][N];
};

// koff / voff: this lane's K / V byte offsets inside a 16-token sub-tile
// (the resources start at the sub-tile).
template <int N>
__device__ __forceinline__ void load_tile(Tile<N>& t, rsrc_t kr, rsrc_t vr, int koff, int voff) {
  constexpr int kRow = 16 * 4 * N;  // bytes per token row = D * elem_bytes
#pragma unroll
  for (int kk = 0; kk < N; ++kk)
    t.k[kk] = __builtin_bit_cast(
        uint4, __builtin_amdgcn_raw_buffer_load_b128(kr, koff + kk * 1024, 0, kStreamPolicy));
#pragma unroll
  for (int e = 0; e < 4; ++e) {
    if constexpr (N == 2) {
      const uint2 x = __builtin_bit_cast(
          uint2, __builtin_amdgcn_raw_buffer_load_b64(vr, voff + e * kRow, 0, kStreamPolicy));
      t.v[e][0] = x.x; t.v[e][1] = x.y;
    } else {
#pragma unroll
      for (int j = 0; j < N / 4; ++j) {
        const uint4 x = __builtin_bit_cast(
            uint4, __builtin_amdgcn_raw_buffer_load_b128(vr, voff + e * kRow + 16 * j, 0,
                                                         kStreamPolicy));
        t.v[e][4 * j + 0] = x.x; t.v[e][4 * j + 1] = x.y;
        t.v[e][4 * j + 2] = x.z; t.v[e][4 * j + 3] = x.w;
      }
    }
  }
}

// Query operand (B of the QK MFMA): lane (r, g) holds query head h*G+g,
// 16-byte chunks r + 4*kk of its row; zero for padding columns.
template <int N>
__device__ __forceinline__ void load_query(uint4 (&qb)[N], const void* q, int s, int h, int G,
                                           int Hq, int lane) {
  constexpr int kRow = 64 * N;
  const int r = lane >> 4, g = lane & 15;
  const char* qrow = static_cast<const char*>(q) +
                     ((size_t)s * Hq + (size_t)h * G + (g < G ? g : 0)) * kRow;
#pragma unroll
  for (int kk = 0; kk < N; ++kk)
    qb[kk] = g < G ? *reinterpret_cast<const uint4*>(qrow + 16 * (r + 4 * kk)) : make_uint4(0, 0, 0, 0);
}

// Per-wave online-softmax state of one item.
template <int kMM>
struct WaveState {
  float m;           // running max of column (lane & 15), base-2 logits
  float l;           // running normaliser of the lane's own tokens
  floatx4 acc[kMM];  // O^T rows (D/16)*(4*(lane>>4)+rr) + mm, column lane & 15
  __device__ __forceinline__ void reset() {
    m = kNegInf;
    l = 0.f;
#pragma unroll
    for (int mm = 0; mm < kMM; ++mm) acc[mm] = floatx4{0.f, 0.f, 0.f, 0.f};
  }
};

// Re-deal a K sub-tile from its load order (lane-contiguous 16-byte chunks)
// into the MFMA A operand order (lane l: token l & 15, chunks (l >> 4) + 4*kk)
// through this wave's LDS slot.  Chunk c of token row t is stored at chunk
// position c ^ (t & mask) so that both the writes and the 16-row reads spread
// over the banks.
template <int N>
__device__ __forceinline__ void restage_k(uint4 (&a)[N], const Tile<N>& t, char* lds, int lane) {
  constexpr int kRow = 64 * N;
  constexpr int kSwz = (4 * N - 1) < 15 ? (4 * N - 1) : 15;
#pragma unroll
  for (int kk = 0; kk < N; ++kk) {
    const int b = 1024 * kk + 16 * lane;
    const int row = b / kRow, c = (b % kRow) / 16;
    *reinterpret_cast<uint4*>(lds + row * kRow + ((c ^ (row & kSwz)) * 16)) = t.k[kk];
  }
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
  __builtin_amdgcn_wave_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
  const int row = lane & 15;
#pragma unroll
  for (int kk = 0; kk < N; ++kk) {
    const int c = (lane >> 4) + 4 * kk;
    a[kk] = *reinterpret_cast<const uint4*>(lds + row * kRow + ((c ^ (row & kSwz)) * 16));
  }
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
  __builtin_amdgcn_wave_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
}

// Maximum of x over the lanes l, l ^ 16, l ^ 32, l ^ 48 (the four row groups
// of one MFMA column): two row swaps (v_permlane16_swap, v_permlane32_swap),
// each one VALU instruction with no LDS round trip.  The NaN-propagating
// maximum needs no quieting of its inputs (fmaxf's NaN rules make the
// compiler add one instruction per operand); logits are finite here.
__device__ __forceinline__ float rows_max(float x) {
  unsigned u = __float_as_uint(x);
  const auto a = __builtin_amdgcn_permlane16_swap(u, u, false, false);
  x = __builtin_elementwise_maximum(__uint_as_float(a[0]), __uint_as_float(a[1]));
  u = __float_as_uint(x);
  const auto b = __builtin_amdgcn_permlane32_swap(u, u, false, false);
  return __builtin_elementwise_maximum(__uint_as_float(b[0]), __uint_as_float(b[1]));
}

// QK, mask, online softmax and PV of one 16-token sub-tile whose K is in the
// MFMA A operand order (ka) and V in its load order (vv); `valid` tokens
// (from the sub-tile's first) are real for this lane's column, the rest are
// masked.
template <int DT, int N, int kMM>
__device__ __forceinline__ void attend_core(const uint4 (&ka)[N], const uint32_t (&vv)[4][N],
                                            const uint4 (&qb)[N], int valid, float scale_log2,
                                            int r, WaveState<kMM>& st) {
  // ---- QK on MFMA ----------------------------------------------------------
  floatx4 S = {0.f, 0.f, 0.f, 0.f};
  if constexpr (DT == DT_F32) {
#pragma unroll
    for (int kk = 0; kk < N; ++kk) {
      S = __builtin_amdgcn_mfma_f32_16x16x4f32(__uint_as_float(ka[kk].x), __uint_as_float(qb[kk].x), S, 0, 0, 0);
      S = __builtin_amdgcn_mfma_f32_16x16x4f32(__uint_as_float(ka[kk].y), __uint_as_float(qb[kk].y), S, 0, 0, 0);
      S = __builtin_amdgcn_mfma_f32_16x16x4f32(__uint_as_float(ka[kk].z), __uint_as_float(qb[kk].z), S, 0, 0, 0);
      S = __builtin_amdgcn_mfma_f32_16x16x4f32(__uint_as_float(ka[kk].w), __uint_as_float(qb[kk].w), S, 0, 0, 0);
    }
  } else if constexpr (DT == DT_F16) {
#pragma unroll
    for (int kk = 0; kk < N; ++kk)
      S = __builtin_amdgcn_mfma_f32_16x16x32_f16(__builtin_bit_cast(halfx8, ka[kk]),
                                                 __builtin_bit_cast(halfx8, qb[kk]), S, 0, 0, 0);
  } else {
#pragma unroll
    for (int kk = 0; kk < N; ++kk)
      S = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, ka[kk]),
                                                  __builtin_bit_cast(bf16x8, qb[kk]), S, 0, 0, 0);
  }

  // ---- mask + online softmax (lane (r, g) holds tokens 4r..4r+3 of column g)
  float sv[4];
#pragma unroll
  for (int e = 0; e < 4; ++e) sv[e] = (4 * r + e < valid) ? S[e] * scale_log2 : kNegInf;
  const auto mx = [](float a, float b) { return __builtin_elementwise_maximum(a, b); };
  const float mloc = rows_max(mx(mx(sv[0], sv[1]), mx(sv[2], sv[3])));
  const float m_new = mx(st.m, mloc);
  const float mb = m_new == kNegInf ? 0.f : m_new;
  const float alpha = fast_exp2(st.m - mb);
  float pe[4];
#pragma unroll
  for (int e = 0; e < 4; ++e) pe[e] = fast_exp2(sv[e] - mb);
  st.l = st.l * alpha + ((pe[0] + pe[1]) + (pe[2] + pe[3]));
  st.m = m_new;
#pragma unroll
  for (int mm = 0; mm < kMM; ++mm) st.acc[mm] *= alpha;

  // Rows at or past `valid` were loaded as zeros (their buffer range ends at
  // the last real token), so stale or NaN bits in unused slots never reach PV.

  // ---- PV on MFMA ----------------------------------------------------------
  if constexpr (DT == DT_F32) {
#pragma unroll
    for (int mm = 0; mm < kMM; ++mm) {
#pragma unroll
      for (int e = 0; e < 4; ++e)
        st.acc[mm] = __builtin_amdgcn_mfma_f32_16x16x4f32(__uint_as_float(vv[e][mm]), pe[e],
                                                          st.acc[mm], 0, 0, 0);
    }
  } else {
    uint2 phi, plo;
    if constexpr (DT == DT_BF16) {
      // hi = truncation to bf16 (exact bits), lo = RNE(p - hi)
      const uint32_t b0 = __float_as_uint(pe[0]), b1 = __float_as_uint(pe[1]);
      const uint32_t b2 = __float_as_uint(pe[2]), b3 = __float_as_uint(pe[3]);
      phi.x = __builtin_amdgcn_perm(b1, b0, 0x07060302u);
      phi.y = __builtin_amdgcn_perm(b3, b2, 0x07060302u);
      const floatx2 l01 = {pe[0] - __uint_as_float(b0 & 0xffff0000u),
                           pe[1] - __uint_as_float(b1 & 0xffff0000u)};
      const floatx2 l23 = {pe[2] - __uint_as_float(b2 & 0xffff0000u),
                           pe[3] - __uint_as_float(b3 & 0xffff0000u)};
      plo.x = __builtin_bit_cast(uint32_t, __builtin_convertvector(l01, bf16x2));
      plo.y = __builtin_bit_cast(uint32_t, __builtin_convertvector(l23, bf16x2));
    } else {
      // hi = round-toward-zero to fp16, lo = the exact remainder rounded again
      const fp16x2 h01 = __builtin_amdgcn_cvt_pkrtz(pe[0], pe[1]);
      const fp16x2 h23 = __builtin_amdgcn_cvt_pkrtz(pe[2], pe[3]);
      phi.x = __builtin_bit_cast(uint32_t, h01);
      phi.y = __builtin_bit_cast(uint32_t, h23);
      const fp16x2 l01 = __builtin_amdgcn_cvt_pkrtz(pe[0] - (float)h01[0], pe[1] - (float)h01[1]);
      const fp16x2 l23 = __builtin_amdgcn_cvt_pkrtz(pe[2] - (float)h23[0], pe[3] - (float)h23[1]);
      plo.x = __builtin_bit_cast(uint32_t, l01);
      plo.y = __builtin_bit_cast(uint32_t, l23);
    }
#pragma unroll
    for (int mm = 0; mm < kMM; ++mm) {
      const uint32_t sel = (mm & 1) ? 0x07060302u : 0x05040100u;
      const int wd = mm >> 1;
      uint2 a;
      a.x = __builtin_amdgcn_perm(vv[1][wd], vv[0][wd], sel);
      a.y = __builtin_amdgcn_perm(vv[3][wd], vv[2][wd], sel);
      if constexpr (DT == DT_BF16) {
        const shortx4 A = __builtin_bit_cast(shortx4, a);
        st.acc[mm] = __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(A, __builtin_bit_cast(shortx4, phi),
                                                               st.acc[mm], 0, 0, 0);
        st.acc[mm] = __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(A, __builtin_bit_cast(shortx4, plo),
                                                               st.acc[mm], 0, 0, 0);
      } else {
        const halfx4 A = __builtin_bit_cast(halfx4, a);
        st.acc[mm] = __builtin_amdgcn_mfma_f32_16x16x16f16(A, __builtin_bit_cast(halfx4, phi),
                                                           st.acc[mm], 0, 0, 0);
        st.acc[mm] = __builtin_amdgcn_mfma_f32_16x16x16f16(A, __builtin_bit_cast(halfx4, plo),
                                                           st.acc[mm], 0, 0, 0);
      }
    }
  }
}

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
                                                float scale_log2, int r, WaveState<kMM>& st) {
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
  const float nmb = st.m == kNegInf ? 0.f : -st.m;
  float pe[8];
#pragma unroll
  for (int e = 0; e < 8; ++e) pe[e] = fast_exp2(__builtin_fmaf(sv[e], scale_log2, nmb));
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

// attend_core for a sub-tile as loaded: K is re-dealt through `lds`, this
// wave's private staging slot (at least one sub-tile of K).
template <int DT, int N, int kMM>
__device__ __forceinline__ void attend_subtile(Tile<N>& t, const uint4 (&qb)[N], int valid,
                                               float scale_log2, int r, WaveState<kMM>& st,
                                               char* lds) {
  uint4 ka[N];
  restage_k<N>(ka, t, lds, threadIdx.x & 63);
  attend_core<DT, N, kMM>(ka, t.v, qb, valid, scale_log2, r, st);
}

template <int DT, int D, int BS>
struct Geometry {
  static constexpr int EB = Elem<DT>::bytes;
  static constexpr int N = D * EB / 64;  // 16-byte K chunks per lane per sub-tile
  static constexpr int kRow = D * EB;    // bytes per token row
  static constexpr int kMM = D / 16;     // PV passes (MFMA row blocks of the head dim)
  static constexpr int kTileBytes = BS * kRow;
  static_assert(kPartitionTokens % BS == 0 && BS % kSub == 0, "partition/block sizes");
};

// Lane (r, g) of a finished wave state holds column g's accumulator rows
// d = (D/16)*(4r + rr) + mm, i.e. the contiguous run d in [r*D/4, (r+1)*D/4)
// in the order idx = rr*(D/16) + mm.  Gather that run.
template <int D, int kMM>
__device__ __forceinline__ void lane_run(float (&o)[D / 4], const WaveState<kMM>& st) {
#pragma unroll
  for (int rr = 0; rr < 4; ++rr)
#pragma unroll
    for (int mm = 0; mm < kMM; ++mm) o[rr * kMM + mm] = st.acc[mm][rr];
}

// Store a lane's run of D/4 values (already scaled) to `dst` (16-byte aligned)
// in the pool dtype, as 16-byte vector stores.
template <int DT, int D>
__device__ __forceinline__ void store_run(void* dst, const float (&o)[D / 4]) {
  if constexpr (DT == DT_F32) {
#pragma unroll
    for (int i = 0; i < D / 16; ++i)
      reinterpret_cast<float4*>(dst)[i] = make_float4(o[4 * i], o[4 * i + 1], o[4 * i + 2], o[4 * i + 3]);
  } else {
    uint32_t packed[D / 8];
#pragma unroll
    for (int i = 0; i < D / 8; ++i) {
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
    for (int i = 0; i < D / 32; ++i)
      reinterpret_cast<uint4*>(dst)[i] =
          make_uint4(packed[4 * i], packed[4 * i + 1], packed[4 * i + 2], packed[4 * i + 3]);
  }
}

// ===========================================================================
// Grid path
// ===========================================================================

// LDS used to merge the four waves' states of one item.  Between merges,
// o[w] is wave w's private K staging slot (at least one 16-token sub-tile of
// K: 16 * D * 4 bytes <= sizeof(o[w])).
template <int D>
struct MergeSmem {
  float ml[kWaves][2][16];
  float o[kWaves][16][D + 4];
};

// Merge the four waves' states of item (s, h, p) and write either the final
// output (single-partition or empty context) or the partition's state.
// Called by the whole workgroup; leaves the LDS free for the next item.
template <int DT, int D, int kMM>
__device__ __forceinline__ void merge_item(MergeSmem<D>& sm, WaveState<kMM>& st, const AttnParams& prm,
                                           int w, int lane, int s, int h, int p, int nparts) {
  const int r = lane >> 4, g = lane & 15;
  const int G = prm.group;
  // column normaliser: sum over the four row groups
  st.l += __shfl_xor(st.l, 16);
  st.l += __shfl_xor(st.l, 32);
  if (g < G) {
    if (r == 0) {
      sm.ml[w][0][g] = st.m;
      sm.ml[w][1][g] = st.l;
    }
#pragma unroll
    for (int mm = 0; mm < kMM; ++mm) {
#pragma unroll
      for (int rr = 0; rr < 4; ++rr) sm.o[w][g][(D / 16) * (4 * r + rr) + mm] = st.acc[mm][rr];
    }
  }
  __syncthreads();
  const int P = prm.max_partitions;
  const int Hq = prm.num_q_heads;
  for (int idx = threadIdx.x; idx < G * D; idx += kThreads) {
    const int gg = idx / D, d = idx % D;
    float M = kNegInf;
#pragma unroll
    for (int ww = 0; ww < kWaves; ++ww) M = fmaxf(M, sm.ml[ww][0][gg]);
    float lsum = 0.f, o = 0.f;
#pragma unroll
    for (int ww = 0; ww < kWaves; ++ww) {
      const float mw = sm.ml[ww][0][gg];
      const float f = mw == kNegInf ? 0.f : fast_exp2(mw - M);
      lsum += f * sm.ml[ww][1][gg];
      o += f * sm.o[ww][gg][d];
    }
    const size_t row = (size_t)s * Hq + (size_t)h * G + gg;
    if (nparts <= 1) {
      store_out<DT>(prm.out, row * D + d, lsum > 0.f ? o / lsum : 0.f);
    } else {
      const size_t prow = row * P + p;
      prm.part_o[prow * D + d] = o;
      if (d == 0) {
        prm.part_ml[prow * 2 + 0] = M;
        prm.part_ml[prow * 2 + 1] = lsum;
      }
    }
  }
  __syncthreads();
}

// One item's coordinates and extent, uniform across the workgroup.
struct Item {
  int s, h, p;
  int ctx;     // context length of sequence s
  int nparts;  // its partitions (0 for an empty context)
  int tok0;    // first token of partition p
  int nsub;    // 16-token sub-tiles holding tokens of this partition
  int niter;   // ring steps per wave: max(1, ceil(nsub / 4))
};

__device__ __forceinline__ Item make_item(int s, int h, int p, int ctx) {
  Item it;
  it.s = s;
  it.h = h;
  it.p = p;
  it.ctx = ctx;
  it.nparts = (ctx + kPartitionTokens - 1) / kPartitionTokens;
  it.tok0 = p * kPartitionTokens;
  int ntok = ctx - it.tok0;
  ntok = ntok < 0 ? 0 : (ntok > kPartitionTokens ? kPartitionTokens : ntok);
  it.nsub = (ntok + kSub - 1) / kSub;
  const int n = (it.nsub + kWaves - 1) / kWaves;
  it.niter = n > 0 ? n : 1;
  return it;
}

// Block ids of a wave's sub-tiles of an item: lane i holds the id for step i
// (sub-tile w + 4i), -1 where that sub-tile holds no token.
template <int BS>
__device__ __forceinline__ int load_ids(const AttnParams& prm, const Item& it, int w, int lane) {
  const int j = w + kWaves * lane;
  int id = -1;
  if (lane < it.niter && j < it.nsub)
    id = prm.block_tables[(size_t)it.s * prm.max_blocks_per_seq + (it.tok0 + kSub * j) / BS];
  return id;
}


// Issue the loads of step i of item `it` for wave w.  The buffer range of a
// sub-tile ends at its last real token, so rows past the context (and a whole
// sub-tile that holds no token or whose block id lies outside the pool) read
// as zeros and touch no memory.
template <int DT, int D, int BS>
__device__ __forceinline__ void issue_step(Tile<Geometry<DT, D, BS>::N>& t, const AttnParams& prm,
                                           const Item& it, int ids, int i, int w, int koff, int voff) {
  using Geo = Geometry<DT, D, BS>;
  const int j = w + kWaves * i;
  int phys = __builtin_amdgcn_readlane(ids, i);
  const bool ok = j < it.nsub && (unsigned)phys < (unsigned)prm.num_blocks;
  phys = ok ? phys : 0;
  int valid = it.ctx - (it.tok0 + kSub * j);
  valid = valid > kSub ? kSub : valid;
  const size_t sub = ((size_t)phys * prm.num_kv_heads + it.h) * Geo::kTileBytes +
                     ((it.tok0 + kSub * j) % BS) * Geo::kRow;
  const int nrec = ok ? valid * Geo::kRow : 0;
  load_tile<Geo::N>(t, make_rsrc(static_cast<const char*>(prm.k_cache) + sub, nrec),
                    make_rsrc(static_cast<const char*>(prm.v_cache) + sub, nrec), koff, voff);
}

// Tokens of step i of item `it` (for wave w) that are real: 0..16.
__device__ __forceinline__ int step_valid(const AttnParams& prm, const Item& it, int ids, int i, int w) {
  const int j = w + kWaves * i;
  const int phys = __builtin_amdgcn_readlane(ids, i);
  if (j >= it.nsub || (unsigned)phys >= (unsigned)prm.num_blocks) return 0;
  const int v = it.ctx - (it.tok0 + kSub * j);
  return v > kSub ? kSub : v;
}

// ---------------------------------------------------------------------------
// Grid kernel: one workgroup per possible item (batches above kMaxStreamSeqs).
// ---------------------------------------------------------------------------

template <int DT, int D, int BS>
__global__ __launch_bounds__(kThreads) __attribute__((amdgpu_waves_per_eu(2)))
void attn_grid_kernel(AttnParams prm) {
  using Geo = Geometry<DT, D, BS>;
  constexpr int N = Geo::N;
  constexpr int kMM = Geo::kMM;
  __shared__ MergeSmem<D> sm;

  const int lane = threadIdx.x & 63;
  const int w = uniform(threadIdx.x >> 6);
  const int r = lane >> 4;

  // Logical order (kv head, partition, sequence): each XCD gets a range of
  // kv heads, and inside it the first partitions of every sequence come
  // before the later ones, so workgroups of short sequences' missing
  // partitions (which exit at once) are dispatched last.
  const int P = prm.max_partitions;
  const int B = prm.num_seqs;
  const int L = xcd_remap(blockIdx.x, gridDim.x);
  const int h = L / (P * B);
  const int p = (L / B) % P;
  const int s = L % B;

  int ctx = prm.context_lens[s];
  ctx = ctx < 0 ? 0 : (ctx > prm.max_context_len ? prm.max_context_len : ctx);
  const Item it = make_item(s, h, p, ctx);
  if (p >= (it.nparts > 0 ? it.nparts : 1)) return;

  const int ids = load_ids<BS>(prm, it, w, lane);
  uint4 qb[N];
  load_query<N>(qb, prm.q, s, h, prm.group, prm.num_q_heads, lane);
  const int koff = 16 * lane;
  char* kst = reinterpret_cast<char*>(&sm.o[w][0][0]);  // this wave's K staging slot
  const int voff = (4 * r) * Geo::kRow + (lane & 15) * (4 * N);
  const float scale_log2 = prm.scale_log2;

  WaveState<kMM> st;
  st.reset();
  auto compute = [&](Tile<N>& t, int i) {
    const int valid = step_valid(prm, it, ids, i, w);
    if (valid > 0) attend_subtile<DT, N, kMM>(t, qb, valid, scale_log2, r, st, kst);
  };
  // 3-deep ring within the item; issue indices are clamped so every slot has
  // the same load count.
  const int last = it.niter - 1;
  Tile<N> t0, t1, t2;
  issue_step<DT, D, BS>(t0, prm, it, ids, 0, w, koff, voff);
  issue_step<DT, D, BS>(t1, prm, it, ids, min(1, last), w, koff, voff);
  int i = 0;
  for (; i + 2 < it.niter; i += 3) {
    issue_step<DT, D, BS>(t2, prm, it, ids, i + 2, w, koff, voff);
    compute(t0, i);
    issue_step<DT, D, BS>(t0, prm, it, ids, min(i + 3, last), w, koff, voff);
    compute(t1, i + 1);
    issue_step<DT, D, BS>(t1, prm, it, ids, min(i + 4, last), w, koff, voff);
    compute(t2, i + 2);
  }
  if (i < it.niter) compute(t0, i);
  if (i + 1 < it.niter) compute(t1, i + 1);
  merge_item<DT, D, kMM>(sm, st, prm, w, lane, s, h, p, it.nparts);
}

// ---------------------------------------------------------------------------
// Merge of the partitions of one (sequence, query head): one wave, lanes over
// the head dim, partitions visited in logical order.
// ---------------------------------------------------------------------------

template <int DT, int D>
__global__ __launch_bounds__(64) void attn_reduce_kernel(AttnParams prm) {
  const int lane = threadIdx.x;
  const int Hq = prm.num_q_heads;
  const int s = blockIdx.x / Hq;
  const int hq = blockIdx.x % Hq;
  int ctx = prm.context_lens[s];
  ctx = ctx < 0 ? 0 : (ctx > prm.max_context_len ? prm.max_context_len : ctx);
  const int nparts = (ctx + kPartitionTokens - 1) / kPartitionTokens;
  if (nparts <= 1) return;
  const int P = prm.max_partitions;
  const size_t base = ((size_t)s * Hq + hq) * P;
  const float* ml = prm.part_ml + base * 2;
  const float* po = prm.part_o + base * D;

  float M = kNegInf;
  for (int p = lane; p < nparts; p += 64) M = fmaxf(M, ml[2 * p]);
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) M = fmaxf(M, __shfl_xor(M, off));

  constexpr int kPer = D / 64;
  float o[kPer];
#pragma unroll
  for (int j = 0; j < kPer; ++j) o[j] = 0.f;
  float lsum = 0.f;
#pragma unroll 4
  for (int p = 0; p < nparts; ++p) {
    const float mp = ml[2 * p];
    const float f = mp == kNegInf ? 0.f : fast_exp2(mp - M);
    lsum += f * ml[2 * p + 1];
#pragma unroll
    for (int j = 0; j < kPer; ++j) o[j] += f * po[(size_t)p * D + lane + 64 * j];
  }
  const float inv = lsum > 0.f ? 1.f / lsum : 0.f;
  const size_t orow = ((size_t)s * Hq + hq) * D;
#pragma unroll
  for (int j = 0; j < kPer; ++j) store_out<DT>(prm.out, orow + lane + 64 * j, o[j] * inv);
}

// ===========================================================================
// Stream path
// ===========================================================================
//
// Columns.  A sequence's MFMA columns are (new token i, query head g) pairs,
// c = i * G + g, cut into groups of 16.  Decode has one new token, so one
// group of G columns.  With L new tokens a sequence has ceil(L * G / 16)
// groups; each group streams the sequence's whole context once.  Column c
// sees logical tokens 0 .. n - L + i (itself and everything before it).

// Per-sequence column geometry, all wave-uniform.
struct SeqCols {
  int n;      // cached tokens
  int L;      // new tokens (query rows)
  int q0;     // first query row
  int ngrp;   // column groups
};

template <bool MULTI>
__device__ __forceinline__ SeqCols seq_cols(const int* sCtx, const int* sQS, const int* sQL, int s,
                                            int G) {
  SeqCols c;
  c.n = uniform(sCtx[s]);
  if constexpr (MULTI) {
    c.q0 = uniform(sQS[s]);
    c.L = uniform(sQL[s]);
    c.ngrp = (c.L * G + kSub - 1) / kSub;
  } else {
    c.q0 = s;
    c.L = c.n > 0 ? 1 : 0;
    c.ngrp = c.L;
  }
  return c;
}

// Where a global position lies: kv head h, sequence s, column group cg, and
// the global positions [A, E) of that (head, sequence, group)'s sub-tiles.
// sS is the LDS prefix of positions per kv head (sS[s] = positions of
// sequences 0..s-1, sS[B] = per-head total); sequence s owns
// [h*per + sS[s], h*per + sS[s+1]), group after group.  Wave-uniform.
struct SeqSpan {
  int h, s, cg;
  int A, E;
};

template <bool MULTI>
__device__ __forceinline__ SeqSpan locate(int p, int per, const int* sS, const int* sCtx, int B) {
  SeqSpan sp;
  sp.h = p / per;
  const int rr = p - sp.h * per;
  // largest s with sS[s] <= rr: skips sequences that own no position
  int a = 0, b = B - 1;
  while (a < b) {
    const int mid = (a + b + 1) >> 1;
    if (uniform(sS[mid]) <= rr) a = mid; else b = mid - 1;
  }
  sp.s = a;
  const int base = sp.h * per + uniform(sS[a]);
  if constexpr (MULTI) {
    const int nsub = (uniform(sCtx[a]) + kSub - 1) / kSub;
    sp.cg = (rr - uniform(sS[a])) / nsub;
    sp.A = base + sp.cg * nsub;
    sp.E = sp.A + nsub;
  } else {
    sp.cg = 0;
    sp.A = base;
    sp.E = sp.h * per + uniform(sS[a + 1]);
  }
  return sp;
}

// The position list [0, total) cut into one chunk per wave: wave v owns
// [v * chunk, min((v + 1) * chunk, total)).  The cut depends only on total
// and the grid, so every piece boundary, and with it the result, is fixed by
// the context lengths.  total <= kMaxStreamPositions (the host routes larger
// calls elsewhere).
__device__ __forceinline__ int stream_chunk(int total, int waves) {
  const int c = total / waves + (total % waves != 0);
  return c < kMinChunk ? kMinChunk : c;
}

// What the compute side needs to know about one issued sub-tile: its global
// position (-1 for a bubble).  Wave-uniform.
struct SlotMeta {
  int p;
};

// Query operand of column group cg (B of the QK MFMA): lane (r, col) holds
// column c = 16*cg + col, i.e. new token c / G of the sequence and query head
// h*G + c % G, 16-byte chunks r + 4*kk of that row; zero for columns past
// the sequence's L*G.
template <int N, bool MULTI>
__device__ __forceinline__ void load_query_cols(uint4 (&qb)[N], const void* q, const SeqCols& sc,
                                                int h, int cg, int G, int Hq, int lane) {
  constexpr int kRow = 64 * N;
  const int r = lane >> 4;
  const int c = cg * kSub + (lane & 15);
  const bool ok = c < sc.L * G;
  const int i = ok ? (MULTI ? c / G : 0) : 0, g = ok ? (MULTI ? c % G : c) : 0;
  const char* qrow = static_cast<const char*>(q) +
                     ((size_t)(sc.q0 + i) * Hq + (size_t)h * G + g) * kRow;
#pragma unroll
  for (int kk = 0; kk < N; ++kk)
    qb[kk] = ok ? *reinterpret_cast<const uint4*>(qrow + 16 * (r + 4 * kk)) : make_uint4(0, 0, 0, 0);
}

// Tokens of sub-tile t that column group cg can see at all (its last
// column's causal limit), 0..16: later rows are not loaded.
__device__ __forceinline__ int group_rows(const SeqCols& sc, int cg, int G, int t) {
  int i_last = (cg * kSub + kSub - 1) / G;
  i_last = i_last < sc.L - 1 ? i_last : sc.L - 1;
  int v = sc.n - sc.L + i_last + 1 - t * kSub;
  return v > kSub ? kSub : v;
}

template <int D>
__device__ __forceinline__ void load_run(const float* src, float (&o)[D / 4]) {
#pragma unroll
  for (int i = 0; i < D / 16; ++i) {
    const float4 x = reinterpret_cast<const float4*>(src)[i];
    o[4 * i] = x.x;
    o[4 * i + 1] = x.y;
    o[4 * i + 2] = x.z;
    o[4 * i + 3] = x.w;
  }
}

template <int DT, int D, int BS, bool MULTI>
__global__ __launch_bounds__(kThreads) __attribute__((amdgpu_waves_per_eu(2)))
void attn_stream_kernel(AttnParams prm) {
  using Geo = Geometry<DT, D, BS>;
  constexpr int N = Geo::N;
  constexpr int kMM = Geo::kMM;
  constexpr int kMaxSeqs = MULTI ? kMaxMultiSeqs : kMaxStreamSeqs;
  // Per-sequence tables: sS [B + 1] position prefix, sCtx [B] context
  // lengths, and with several new tokens sQS [B] first query row, sQL [B]
  // query rows.  Once every wave has left its loop the same memory carries
  // the waves' first-piece states (sX).
  constexpr int kTabInts = 2 * kMaxSeqs + 1 + (MULTI ? 2 * kMaxSeqs : 0);
  __shared__ __attribute__((aligned(16))) int sTab[kTabInts];
  static_assert(kWaves * 64 * (D / 4) * sizeof(float) <= kTabInts * sizeof(int),
                "first-piece states fit the tables");
  int* const sS = sTab;
  int* const sCtx = sTab + kMaxSeqs + 1;
  int* const sQS = sCtx + kMaxSeqs;
  int* const sQL = sQS + (MULTI ? kMaxSeqs : 0);
  __shared__ int sScan[kWaves];
  __shared__ __attribute__((aligned(16))) char sK[kWaves][kSub * Geo::kRow];
  // The chunk's last piece, when partial, is parked in LDS as it finishes:
  // 16-byte chunks i < kInK of each lane's run in the wave's K staging slot
  // (no longer needed then), the rest in sX1.
  constexpr int kRunChunks = D / 16;
  constexpr int kInK = (int)(sizeof(sK[0]) / (64 * 16)) < kRunChunks ? (int)(sizeof(sK[0]) / (64 * 16))
                                                                      : kRunChunks;
  __shared__ __attribute__((aligned(16))) float4 sX1[kWaves][(kRunChunks - kInK) * 64 + 1];
  __shared__ float2 sML[2][kWaves][kSub];  // (max, normaliser) per column: first, last piece
  __shared__ int sInfo[2][kWaves][6];      // span of the first / last piece: A, E, h, cg, q0, L

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int w = uniform(tid >> 6);
  const int r = lane >> 4;
  const int B = prm.num_seqs;
  const int G = prm.group;
  const int Hq = prm.num_q_heads;

  // ---- per-sequence tables and the position prefix (every workgroup, LDS) ---
  // Multi-token: query rows [query_start[s], query_start[s+1]) clamped to
  // [0, num_query_tokens], and at most min(n, max_query_len) of them, so that
  // no index derived from them leaves its buffer whatever the metadata holds.
  const int per_thread = (B + kThreads - 1) / kThreads;
  int mine = 0;
  for (int k = 0; k < per_thread; ++k) {
    const int s = tid * per_thread + k;
    if (s < B) {
      int c = prm.context_lens[s];
      c = c < 0 ? 0 : (c > prm.max_context_len ? prm.max_context_len : c);
      int groups = c > 0 ? 1 : 0;
      if constexpr (MULTI) {
        const int T = prm.num_query_tokens;
        int q0 = prm.query_start[s], qe = prm.query_start[s + 1];
        q0 = q0 < 0 ? 0 : (q0 > T ? T : q0);
        qe = qe < q0 ? q0 : (qe > T ? T : qe);
        int L = qe - q0;
        L = L < c ? L : c;
        L = L < prm.max_query_len ? L : prm.max_query_len;
        sQS[s] = q0;
        sQL[s] = L;
        groups = (L * G + kSub - 1) / kSub;
      }
      sCtx[s] = c;
      mine += groups * ((c + kSub - 1) / kSub);
    }
  }
  int incl = mine;
#pragma unroll
  for (int off = 1; off < 64; off <<= 1) {
    const int y = __shfl_up(incl, off);
    if (lane >= off) incl += y;
  }
  if (lane == 63) sScan[w] = incl;
  __syncthreads();
  int run = incl - mine;
  for (int ww = 0; ww < w; ++ww) run += sScan[ww];
  for (int k = 0; k < per_thread; ++k) {
    const int s = tid * per_thread + k;
    if (s < B) {
      sS[s] = run;
      int groups = sCtx[s] > 0 ? 1 : 0;
      if constexpr (MULTI) groups = (sQL[s] * G + kSub - 1) / kSub;
      run += groups * ((sCtx[s] + kSub - 1) / kSub);
    }
  }
  if (tid == 0) sS[B] = sScan[0] + sScan[1] + sScan[2] + sScan[3];
  __syncthreads();
  if (blockIdx.x == 0)  // for the merge kernel
    for (int s = tid; s <= B; s += kThreads) prm.seq_prefix[s] = sS[s];

  // ---- this wave's chunk of positions -----------------------------------------
  const int per = uniform(sS[B]);  // positions per kv head
  const int total = prm.num_kv_heads * per;
  const int chunk = stream_chunk(total, (int)gridDim.x * kWaves);
  const int wg = xcd_remap(blockIdx.x, gridDim.x);
  const int wv = wg * kWaves + w;
  // end of wave v's chunk (v = kWaves * wg + i); the workgroup's positions
  // are [ga, end of wave kWaves * wg + kWaves - 1)
  auto chunk_end = [&](int v) -> int { return (int)min((long long)(v + 1) * chunk, (long long)total); };
  const int a = (int)min((long long)wv * chunk, (long long)total);
  const int b = chunk_end(wv);
  const int ga = (int)min((long long)wg * kWaves * chunk, (long long)total);

  const int koff = 16 * lane;
  const int voff = (4 * r) * Geo::kRow + (lane & 15) * (4 * N);
  char* kst = sK[w];
  const float scale_log2 = prm.scale_log2;

  // ---- issue cursor: next position whose tiles are loaded ---------------------
  int pi = a;
  SeqSpan si;
  SeqCols ci;
  // Block ids are read one at a time with scalar loads through the constant
  // address space: the index is wave-uniform, the row stays in the scalar
  // cache, and the scalar counter keeps the vector loads of the tiles in
  // flight (a vector load of the ids, used right away, drained them).
  typedef const __attribute__((address_space(4))) int32_t const_i32;
  const_i32* row_i = nullptr;
  auto enter_issue_seq = [&]() {
    si = locate<MULTI>(pi, per, sS, sCtx, B);
    ci = seq_cols<MULTI>(sCtx, sQS, sQL, si.s, G);
    row_i = (const_i32*)prm.block_tables + (size_t)si.s * prm.max_blocks_per_seq;
  };
  auto issue = [&](Tile<N>& t, SlotMeta& m) {
    if (pi < b) {
      m.p = pi;
      // all wave-uniform; readfirstlane keeps them (and the resources built
      // from them) in scalar registers
      const int tsub = uniform(pi - si.A);
      // blk < ceil(n / BS) <= max_blocks_per_seq: inside the sequence's row
      const int blk = tsub * kSub / BS;
      int phys = row_i[blk];
      const bool ok = (unsigned)phys < (unsigned)prm.num_blocks;
      phys = ok ? phys : 0;
      int rows;
      if constexpr (MULTI) {
        rows = group_rows(ci, uniform(si.cg), G, tsub);
      } else {
        rows = ci.n - tsub * kSub;
        rows = rows > kSub ? kSub : rows;
      }
      const size_t sub = ((size_t)phys * prm.num_kv_heads + uniform(si.h)) * Geo::kTileBytes +
                         (tsub * kSub % BS) * Geo::kRow;
      // the range ends at the last row any column can see: later rows, and
      // every row of a block id outside the pool, read as zeros without
      // touching memory
      const int nrec = uniform(ok && rows > 0 ? rows * Geo::kRow : 0);
      load_tile<N>(t, make_rsrc(static_cast<const char*>(prm.k_cache) + sub, nrec),
                   make_rsrc(static_cast<const char*>(prm.v_cache) + sub, nrec), koff, voff);
      ++pi;
      if (pi < b && pi == si.E) enter_issue_seq();
    } else {
      // past the chunk: keep the per-slot load count fixed, touch no memory
      m.p = -1;
      load_tile<N>(t, make_rsrc(prm.k_cache, 0), make_rsrc(prm.v_cache, 0), koff, voff);
    }
  };

  // ---- compute cursor -----------------------------------------------------------
  // The open piece: positions [p0, ...) of group span sc.  A piece that covers
  // its whole group is written to `out` at once.  Otherwise it is the chunk's
  // first piece or its last one (ending at b), and nothing of it goes to
  // global memory inside the loop: stores share the vector memory counter
  // with loads and it retires in order, so a store issued mid-stream makes
  // every tile load issued after it wait for the store's acknowledgement.
  // The first piece's run stays in registers (fp32 at D = 128, whose wider
  // tiles leave no room, parks it in this wave's workspace row instead); the
  // last piece's run goes to LDS.  The spans' identities go to sInfo.
  constexpr bool kHold = !(DT == DT_F32 && D > 64);
  const int cols = prm.slot_cols;
  const int col = lane & 15;
  bool open = false;
  int p0 = 0;
  SeqSpan sc;
  SeqCols cc;
  int vis_c = 0;  // this lane's column: tokens it can see (0 for a padding column)
  uint4 qb[N];
  WaveState<kMM> st;
  float o0[D / 4];  // the first piece's run
  float m0 = 0.f, l0 = 0.f;
  bool has0 = false, has1 = false;
  float* const park = prm.part_o + (((size_t)gridDim.x * 2 + wv) * cols + (col < cols ? col : 0)) * D +
                      r * (D / 4);
  auto x1_chunk = [&](int i) -> float4& {
    return i < kInK ? reinterpret_cast<float4*>(sK[w])[i * 64 + lane] : sX1[w][(i - kInK) * 64 + lane];
  };
  // normalise a group's finished state and write its rows
  auto write_out = [&](float (&o)[D / 4], float l, int h, int cg, int q0, int L, int col, int r) {
    const int c = cg * kSub + col;
    if (c < L * G) {
      const size_t row = MULTI ? (size_t)(q0 + c / G) * Hq + (size_t)h * G + c % G
                               : (size_t)q0 * Hq + (size_t)h * G + c;
      const float inv = l > 0.f ? 1.f / l : 0.f;
#pragma unroll
      for (int i = 0; i < D / 4; ++i) o[i] *= inv;
      store_run<DT, D>(static_cast<char*>(prm.out) + (row * D + r * (D / 4)) * Geo::EB, o);
    }
  };
  auto note_span = [&](int k) {
    if (lane == 0) {
      sInfo[k][w][0] = sc.A;
      sInfo[k][w][1] = sc.E;
      sInfo[k][w][2] = sc.h;
      sInfo[k][w][3] = sc.cg;
      sInfo[k][w][4] = cc.q0;
      sInfo[k][w][5] = cc.L;
    }
  };
  auto finish_piece = [&](int p_end) {
    float l = st.l + __shfl_xor(st.l, 16);
    l += __shfl_xor(l, 32);
    float o[D / 4];
    lane_run<D, kMM>(o, st);
    if (p0 == sc.A && p_end == sc.E) {
      write_out(o, l, sc.h, sc.cg, cc.q0, cc.L, col, r);
    } else if (p0 == a) {
#pragma unroll
      for (int i = 0; i < D / 4; ++i) o0[i] = o[i];
      m0 = st.m;
      l0 = l;
      has0 = true;
      note_span(0);
      if constexpr (!kHold)
        if (col < cols) store_run<DT_F32, D>(park, o0);
    } else {  // only the chunk's last piece can be partial without starting it
#pragma unroll
      for (int i = 0; i < D / 16; ++i)
        x1_chunk(i) = make_float4(o[4 * i], o[4 * i + 1], o[4 * i + 2], o[4 * i + 3]);
      if (r == 0) sML[1][w][col] = make_float2(st.m, l);
      has1 = true;
      note_span(1);
    }
  };
  auto step = [&](Tile<N>& t, const SlotMeta& m) {
    if (!open) {
      sc = locate<MULTI>(m.p, per, sS, sCtx, B);
      cc = seq_cols<MULTI>(sCtx, sQS, sQL, sc.s, G);
      p0 = m.p;
      load_query_cols<N, MULTI>(qb, prm.q, cc, sc.h, sc.cg, G, Hq, lane);
      // Take the wait for the query here, where a piece opens: the loads are
      // conditional, and a wait placed at their use would drain every
      // sub-tile's prefetched loads on every step.
#pragma unroll
      for (int kk = 0; kk < N; ++kk) {
        u32x4 qv = __builtin_bit_cast(u32x4, qb[kk]);
        asm volatile("" : "+v"(qv));
        qb[kk] = __builtin_bit_cast(uint4, qv);
      }
      if constexpr (MULTI) {
        const int c = sc.cg * kSub + (lane & 15);
        vis_c = c < cc.L * G ? cc.n - cc.L + c / G + 1 : 0;
      }
      st.reset();
      open = true;
    }
    const int tsub = m.p - sc.A;
    // real tokens of the sub-tile for this lane's column: in decode every
    // column sees the whole context (padding columns have q = 0 and are
    // never written), so the count is wave-uniform
    int valid = (MULTI ? vis_c : cc.n) - tsub * kSub;
    valid = valid > kSub ? kSub : valid;
    attend_subtile<DT, N, kMM>(t, qb, valid, scale_log2, r, st, kst);
    if (m.p + 1 == sc.E || m.p + 1 == b) {
      finish_piece(m.p + 1);
      open = false;
    }
  };

  if (a < b) {
    enter_issue_seq();
    Tile<N> t0, t1, t2;
    SlotMeta m0, m1, m2;
    issue(t0, m0);
    issue(t1, m1);
    for (;;) {
      issue(t2, m2);
      if (m0.p < 0) break;
      step(t0, m0);
      issue(t0, m0);
      if (m1.p < 0) break;
      step(t1, m1);
      issue(t1, m1);
      if (m2.p < 0) break;
      step(t2, m2);
    }
  }

  // ---- the workgroup's pieces ---------------------------------------------------
  // The four waves hold consecutive chunks.  A group span that crosses a
  // chunk boundary inside the workgroup is merged here, in logical order, by
  // the wave that holds its first piece in the workgroup: a span that starts
  // and ends inside the workgroup is written to `out`; otherwise the merged
  // piece goes to the workgroup's slot 0 (the span starts at or before the
  // workgroup's first position) or slot 1, and the merge kernel finishes it.
  __syncthreads();  // every wave has left its loop: the tables are free
  // The lane index again, opaque to the compiler: addresses derived from it
  // below are not hoisted above the loop, where they would stay live in
  // registers the loop needs.
  int ln = lane;
  asm volatile("" : "+v"(ln));
  const int lcol = ln & 15, lr = ln >> 4;
  float4* const sX0 = reinterpret_cast<float4*>(sTab);  // first pieces: [kWaves][D/16][64 lanes]
  if (has0) {
    if constexpr (!kHold)
      if (lcol < cols) load_run<D>(park, o0);
#pragma unroll
    for (int i = 0; i < D / 16; ++i)
      sX0[(w * (D / 16) + i) * 64 + ln] = make_float4(o0[4 * i], o0[4 * i + 1], o0[4 * i + 2],
                                                        o0[4 * i + 3]);
    if (lr == 0) sML[0][w][lcol] = make_float2(m0, l0);
  }
  __syncthreads();
  // o, m, l: the state of a piece ending at this wave's chunk end (k: which
  // piece, for its span); merges the next waves' first pieces while the span
  // goes on, then writes the result
  auto finish_span = [&](float (&o)[D / 4], float m, float l, int k) {
    const int A = uniform(sInfo[k][w][0]), E = uniform(sInfo[k][w][1]);
    int v = w;
    int bv = b;
    while (E > bv && v + 1 < kWaves) {  // the next wave's first piece continues it
      ++v;
      bv = chunk_end(wg * kWaves + v);
      const float2 ml = sML[0][v][lcol];
      const float M = fmaxf(m, ml.x);
      const float fa = m == kNegInf ? 0.f : fast_exp2(m - M);
      const float fb = ml.x == kNegInf ? 0.f : fast_exp2(ml.x - M);
      l = fa * l + fb * ml.y;
      m = M;
#pragma unroll
      for (int i = 0; i < D / 16; ++i) {
        const float4 x = sX0[(v * (D / 16) + i) * 64 + ln];
        o[4 * i] = fa * o[4 * i] + fb * x.x;
        o[4 * i + 1] = fa * o[4 * i + 1] + fb * x.y;
        o[4 * i + 2] = fa * o[4 * i + 2] + fb * x.z;
        o[4 * i + 3] = fa * o[4 * i + 3] + fb * x.w;
      }
    }
    if (A >= ga && E <= bv) {
      write_out(o, l, uniform(sInfo[k][w][2]), uniform(sInfo[k][w][3]), uniform(sInfo[k][w][4]),
                uniform(sInfo[k][w][5]), lcol, lr);
    } else if (lcol < cols) {  // slot rows of columns >= cols lie past the slot
      const size_t slot = (size_t)wg * 2 + (A <= ga ? 0 : 1);
      store_run<DT_F32, D>(prm.part_o + (slot * cols + lcol) * D + lr * (D / 4), o);
      if (lr == 0) *reinterpret_cast<float2*>(prm.part_ml + (slot * cols + lcol) * 2) = make_float2(m, l);
    }
  };
  // a first piece that started before this chunk belongs to the previous
  // wave's span, unless this wave starts the workgroup
  // (each state is read back from LDS: taking the first piece's registers
  // here instead would make the loop above spill)
  auto own_state = [&](int k, float (&o)[D / 4]) -> float2 {
#pragma unroll
    for (int i = 0; i < D / 16; ++i) {
      const float4 x = k == 0 ? sX0[(w * (D / 16) + i) * 64 + ln]
                     : i < kInK ? reinterpret_cast<const float4*>(sK[w])[i * 64 + ln]
                                : sX1[w][(i - kInK) * 64 + ln];
      o[4 * i] = x.x;
      o[4 * i + 1] = x.y;
      o[4 * i + 2] = x.z;
      o[4 * i + 3] = x.w;
    }
    return sML[k][w][lcol];
  };
  if (has0 && (w == 0 || uniform(sInfo[0][w][0]) >= a)) {
    float o[D / 4];
    const float2 ml = own_state(0, o);
    finish_span(o, ml.x, ml.y, 0);
  }
  if (has1) {
    float o[D / 4];
    const float2 ml = own_state(1, o);
    finish_span(o, ml.x, ml.y, 1);
  }
}

// Merge of the pieces of one split (sequence, kv head, column group) for one
// column: one wave, lanes over the head dim, pieces visited in logical order.
// Grid: sequence x kv head x group (up to the call's maximum) x column.  In
// decode it also writes the zero row of an empty context.
template <int DT, int D, bool MULTI>
__global__ __launch_bounds__(64) void attn_stream_merge_kernel(AttnParams prm) {
  const int lane = threadIdx.x;
  const int Hq = prm.num_q_heads;
  const int G = prm.group;
  const int cols = prm.slot_cols;
  const int ngmax = prm.max_groups;
  int id = blockIdx.x;
  const int col = id % cols;
  id /= cols;
  const int cg = id % ngmax;
  id /= ngmax;
  const int h = id % prm.num_kv_heads;
  const int s = id / prm.num_kv_heads;
  constexpr int kPer = D / 64;
  int ctx = prm.context_lens[s];
  ctx = ctx < 0 ? 0 : (ctx > prm.max_context_len ? prm.max_context_len : ctx);
  int q0 = s, L = ctx > 0 ? 1 : 0;
  if constexpr (MULTI) {
    const int T = prm.num_query_tokens;
    q0 = prm.query_start[s];
    int qe = prm.query_start[s + 1];
    q0 = q0 < 0 ? 0 : (q0 > T ? T : q0);
    qe = qe < q0 ? q0 : (qe > T ? T : qe);
    L = qe - q0;
    L = L < ctx ? L : ctx;
    L = L < prm.max_query_len ? L : prm.max_query_len;
  } else if (ctx == 0) {
    const size_t orow = ((size_t)s * Hq + (size_t)h * G + col) * D;
#pragma unroll
    for (int j = 0; j < kPer; ++j) store_out<DT>(prm.out, orow + lane + 64 * j, 0.f);
    return;
  }
  const int c = cg * kSub + col;
  if (c >= L * G) return;
  const size_t orow = ((size_t)(q0 + c / G) * Hq + (size_t)h * G + c % G) * D;
  const int per = prm.seq_prefix[prm.num_seqs];
  // a workgroup's positions: kWaves consecutive wave chunks
  const int chunk = kWaves * stream_chunk(prm.num_kv_heads * per, prm.stream_wgs * kWaves);
  const int nsub = (ctx + kSub - 1) / kSub;
  const int A = h * per + prm.seq_prefix[s] + cg * nsub;
  const int E = A + nsub;
  const int k1 = A / chunk, k2 = (E - 1) / chunk;
  if (k1 == k2) return;  // one workgroup covered it and wrote `out`
  // workgroup k's piece sits in its slot 0 unless the group starts inside
  // the positions of workgroup k1
  const int first_slot = k1 * 2 + (A != k1 * chunk ? 1 : 0);
  auto row_of = [&](int k) -> size_t { return (size_t)(k == k1 ? first_slot : k * 2) * cols + col; };

  float M = kNegInf;
  for (int k = k1 + lane; k <= k2; k += 64) M = fmaxf(M, prm.part_ml[row_of(k) * 2]);
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) M = fmaxf(M, __shfl_xor(M, off));

  float o[kPer];
#pragma unroll
  for (int j = 0; j < kPer; ++j) o[j] = 0.f;
  float lsum = 0.f;
#pragma unroll 4
  for (int k = k1; k <= k2; ++k) {
    const size_t row = row_of(k);
    const float2 ml = *reinterpret_cast<const float2*>(prm.part_ml + row * 2);
    const float f = ml.x == kNegInf ? 0.f : fast_exp2(ml.x - M);
    lsum += f * ml.y;
#pragma unroll
    for (int j = 0; j < kPer; ++j) o[j] += f * prm.part_o[row * D + lane + 64 * j];
  }
  const float inv = lsum > 0.f ? 1.f / lsum : 0.f;
#pragma unroll
  for (int j = 0; j < kPer; ++j) store_out<DT>(prm.out, orow + lane + 64 * j, o[j] * inv);
}

// The same merge for calls whose partial slots hold 16 columns (several new
// tokens per sequence): one wave per (sequence, kv head, column group), lane
// (r, col) holding column col's run d in [r*D/4, (r+1)*D/4) exactly as the
// stream kernel stores it; the workgroups' pieces are folded in logical order
// with a running max.  (With fewer columns most lanes would idle and a
// group's pieces would be fetched one after another: the per-column kernel
// is faster there.)  Grid: sequence x kv head x group (up to the call's
// maximum).
template <int DT, int D, bool MULTI>
__global__ __launch_bounds__(64) void attn_stream_merge_group_kernel(AttnParams prm) {
  using Geo = Geometry<DT, D, 16>;
  const int lane = threadIdx.x;
  const int r = lane >> 4, col = lane & 15;
  const int Hq = prm.num_q_heads;
  const int G = prm.group;
  const int cols = prm.slot_cols;
  const int ngmax = prm.max_groups;
  int id = blockIdx.x;
  const int cg = id % ngmax;
  id /= ngmax;
  const int h = id % prm.num_kv_heads;
  const int s = id / prm.num_kv_heads;
  int ctx = prm.context_lens[s];
  ctx = ctx < 0 ? 0 : (ctx > prm.max_context_len ? prm.max_context_len : ctx);
  int q0 = s, L = ctx > 0 ? 1 : 0;
  if constexpr (MULTI) {
    const int T = prm.num_query_tokens;
    q0 = prm.query_start[s];
    int qe = prm.query_start[s + 1];
    q0 = q0 < 0 ? 0 : (q0 > T ? T : q0);
    qe = qe < q0 ? q0 : (qe > T ? T : qe);
    L = qe - q0;
    L = L < ctx ? L : ctx;
    L = L < prm.max_query_len ? L : prm.max_query_len;
  } else if (ctx == 0) {
    if (col < G) {
      float z[D / 4];
#pragma unroll
      for (int i = 0; i < D / 4; ++i) z[i] = 0.f;
      store_run<DT, D>(static_cast<char*>(prm.out) +
                           ((((size_t)s * Hq + (size_t)h * G + col) * D) + r * (D / 4)) * Geo::EB,
                       z);
    }
    return;
  }
  const int c = cg * kSub + col;
  if (c >= L * G || col >= cols) return;  // no cross-lane step follows
  const int per = prm.seq_prefix[prm.num_seqs];
  // a workgroup's positions: kWaves consecutive wave chunks
  const int chunk = kWaves * stream_chunk(prm.num_kv_heads * per, prm.stream_wgs * kWaves);
  const int nsub = (ctx + kSub - 1) / kSub;
  const int A = h * per + prm.seq_prefix[s] + cg * nsub;
  const int E = A + nsub;
  const int k1 = A / chunk, k2 = (E - 1) / chunk;
  if (k1 == k2) return;  // one workgroup covered it and wrote `out`
  // workgroup k's piece sits in its slot 0 unless the group starts inside
  // the positions of workgroup k1
  const int first_slot = k1 * 2 + (A != k1 * chunk ? 1 : 0);
  float M = kNegInf, lsum = 0.f;
  float o[D / 4];
#pragma unroll
  for (int i = 0; i < D / 4; ++i) o[i] = 0.f;
#pragma unroll 2
  for (int k = k1; k <= k2; ++k) {
    const size_t row = (size_t)(k == k1 ? first_slot : k * 2) * cols + col;
    const float2 ml = *reinterpret_cast<const float2*>(prm.part_ml + row * 2);
    float x[D / 4];
    load_run<D>(prm.part_o + row * D + r * (D / 4), x);
    const float Mn = fmaxf(M, ml.x);
    const float fa = M == kNegInf ? 0.f : fast_exp2(M - Mn);
    const float fb = ml.x == kNegInf ? 0.f : fast_exp2(ml.x - Mn);
    lsum = fa * lsum + fb * ml.y;
#pragma unroll
    for (int i = 0; i < D / 4; ++i) o[i] = fa * o[i] + fb * x[i];
    M = Mn;
  }
  const float inv = lsum > 0.f ? 1.f / lsum : 0.f;
#pragma unroll
  for (int i = 0; i < D / 4; ++i) o[i] *= inv;
  const size_t orow = (size_t)(q0 + c / G) * Hq + (size_t)h * G + c % G;
  store_run<DT, D>(static_cast<char*>(prm.out) + (orow * D + r * (D / 4)) * Geo::EB, o);
}

// ===========================================================================
// Launch
// ===========================================================================

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

template <int DT, int D, int BS, int GW>
__global__ __launch_bounds__(kThreads) __attribute__((amdgpu_waves_per_eu(GW == 2 ? 2 : 3)))
void attn_prefill_kernel(AttnParams prm) {
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
                                             valid_of(g, sub + 1), scale_log2, r, st[g]);
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
    for (int g = 0; g < kGW; ++g) st[g].reset();
    Tile<N> t;
    load_sub(t, st0 * kWaves + w);
    park(t, 0, exact);
    __syncthreads();
    for (int sg = st0; sg < st1; ++sg) {
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

// Merge of a split prefill context for one (query row, query head): one
// wave, lanes over the head dim, parts in order.  Grid: sequence x new token
// (up to max_query_len) x query head, a wave each, four per workgroup.  The
// number of non-empty parts follows from the same stage counts the prefill
// kernel uses.
template <int DT, int D>
__global__ __launch_bounds__(kThreads) void attn_prefill_merge_kernel(AttnParams prm) {
  const int lane = threadIdx.x & 63;
  const long long id = (long long)blockIdx.x * kWaves + (threadIdx.x >> 6);
  const int Hq = prm.num_q_heads;
  const int G = prm.group;
  const int P = prm.prefill_parts;
  const int hq = (int)(id % Hq);
  const long long rest = id / Hq;
  const int i = (int)(rest % prm.max_query_len);
  const int s = (int)(rest / prm.max_query_len);
  if (s >= prm.num_seqs) return;
  int n = prm.context_lens[s];
  n = n < 0 ? 0 : (n > prm.max_context_len ? prm.max_context_len : n);
  const int T = prm.num_query_tokens;
  int q0 = prm.query_start[s], qe = prm.query_start[s + 1];
  q0 = q0 < 0 ? 0 : (q0 > T ? T : q0);
  qe = qe < q0 ? q0 : (qe > T ? T : qe);
  int L = qe - q0;
  L = L < n ? L : n;
  L = L < prm.max_query_len ? L : prm.max_query_len;
  if (i >= L) return;
  const int kGB = kWaves * prm.prefill_wave_groups;  // groups per column block
  const int c = i * G + hq % G;  // the column, in its kv head's block
  const int cb = c / (kGB * kSub);
  const int ngrp = (L * G + kSub - 1) / kSub;
  const int cg_last = (cb + 1) * kGB < ngrp ? (cb + 1) * kGB - 1 : ngrp - 1;
  int i_last = (cg_last * kSub + kSub - 1) / G;
  i_last = i_last < L - 1 ? i_last : L - 1;
  const int rows_b = n - L + i_last + 1;
  const int nstage_all = ((rows_b + kSub - 1) / kSub + kWaves - 1) / kWaves;
  const int per_part = (nstage_all + P - 1) / P;
  const int nparts = (nstage_all + per_part - 1) / per_part;
  const size_t base = ((size_t)(q0 + i) * Hq + hq) * P;
  constexpr int kPer = D / 64;

  float M = kNegInf;
  for (int k = lane; k < nparts; k += 64) M = fmaxf(M, prm.part_ml[(base + k) * 2]);
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) M = fmaxf(M, __shfl_xor(M, off));
  float o[kPer];
#pragma unroll
  for (int j = 0; j < kPer; ++j) o[j] = 0.f;
  float lsum = 0.f;
  for (int k = 0; k < nparts; ++k) {
    const float2 ml = *reinterpret_cast<const float2*>(prm.part_ml + (base + k) * 2);
    const float f = ml.x == kNegInf ? 0.f : fast_exp2(ml.x - M);
    lsum += f * ml.y;
#pragma unroll
    for (int j = 0; j < kPer; ++j) o[j] += f * prm.part_o[(base + k) * D + lane + 64 * j];
  }
  const float inv = lsum > 0.f ? 1.f / lsum : 0.f;
  const size_t orow = ((size_t)(q0 + i) * Hq + hq) * D;
#pragma unroll
  for (int j = 0; j < kPer; ++j) store_out<DT>(prm.out, orow + lane + 64 * j, o[j] * inv);
}

template <int DT, int D, int BS>
hipError_t launch_typed(const AttnParams& prm, hipStream_t stream) {
  const dim3 block(kThreads);
  const long long nout = (long long)prm.num_seqs * prm.num_q_heads;
  if (nout > 0x7fffffffLL) return hipErrorInvalidConfiguration;
  if (prm.prefill_blocks > 0) {
    const long long nx = (long long)prm.prefill_blocks * prm.prefill_parts;
    if (!prm.query_start || prm.num_seqs > 65535 || prm.num_kv_heads > 65535 ||
        prm.prefill_parts < 1 || nx > 0x7fffffffLL)
      return hipErrorInvalidConfiguration;
    const dim3 grid((unsigned)nx, (unsigned)prm.num_kv_heads, (unsigned)prm.num_seqs);
    if (prm.prefill_wave_groups == 1)
      hipLaunchKernelGGL((attn_prefill_kernel<DT, D, BS, 1>), grid, block, 0, stream, prm);
    else if constexpr (DT != DT_F32)
      hipLaunchKernelGGL((attn_prefill_kernel<DT, D, BS, 2>), grid, block, 0, stream, prm);
    else
      return hipErrorInvalidValue;
    hipError_t err = hipGetLastError();
    if (err != hipSuccess || prm.prefill_parts == 1) return err;
    const long long waves = (long long)prm.num_seqs * prm.max_query_len * prm.num_q_heads;
    const long long nm = (waves + kWaves - 1) / kWaves;
    if (nm > 0x7fffffffLL) return hipErrorInvalidConfiguration;
    hipLaunchKernelGGL((attn_prefill_merge_kernel<DT, D>), dim3((unsigned)nm), block, 0, stream,
                       prm);
    return hipGetLastError();
  }
  if (prm.stream_wgs > 0) {
    const long long ngroups = (long long)prm.num_seqs * prm.num_kv_heads * prm.max_groups;
    const long long nmerge = ngroups * prm.slot_cols;
    if (nmerge > 0x7fffffffLL) return hipErrorInvalidConfiguration;
    if (prm.query_start) {
      hipLaunchKernelGGL((attn_stream_kernel<DT, D, BS, true>), dim3((unsigned)prm.stream_wgs),
                         block, 0, stream, prm);
      hipError_t err = hipGetLastError();
      if (err != hipSuccess) return err;
      if (prm.slot_cols == kSub)
        hipLaunchKernelGGL((attn_stream_merge_group_kernel<DT, D, true>), dim3((unsigned)ngroups),
                           dim3(64), 0, stream, prm);
      else
        hipLaunchKernelGGL((attn_stream_merge_kernel<DT, D, true>), dim3((unsigned)nmerge), dim3(64),
                           0, stream, prm);
      return hipGetLastError();
    }
    hipLaunchKernelGGL((attn_stream_kernel<DT, D, BS, false>), dim3((unsigned)prm.stream_wgs),
                       block, 0, stream, prm);
    hipError_t err = hipGetLastError();
    if (err != hipSuccess) return err;
    hipLaunchKernelGGL((attn_stream_merge_kernel<DT, D, false>), dim3((unsigned)nmerge), dim3(64),
                       0, stream, prm);
    return hipGetLastError();
  }
  if (prm.query_start) return hipErrorInvalidValue;  // multi-token calls take the stream path
  const long long nwg = (long long)prm.num_seqs * prm.num_kv_heads * prm.max_partitions;
  if (nwg <= 0) return hipSuccess;
  if (nwg > 0x7fffffffLL) return hipErrorInvalidConfiguration;
  hipLaunchKernelGGL((attn_grid_kernel<DT, D, BS>), dim3((unsigned)nwg), block, 0, stream, prm);
  hipError_t err = hipGetLastError();
  if (err != hipSuccess || prm.max_partitions <= 1) return err;
  hipLaunchKernelGGL((attn_reduce_kernel<DT, D>), dim3((unsigned)nout), dim3(64), 0, stream, prm);
  return hipGetLastError();
}

template <int DT, int D>
hipError_t launch_bs(const AttnParams& prm, int bs, hipStream_t stream) {
  switch (bs) {
    case 16: return launch_typed<DT, D, 16>(prm, stream);
    case 32: return launch_typed<DT, D, 32>(prm, stream);
    default: return hipErrorInvalidValue;
  }
}

template <int DT>
hipError_t launch_d(const AttnParams& prm, int d, int bs, hipStream_t stream) {
  switch (d) {
    case 64: return launch_bs<DT, 64>(prm, bs, stream);
    case 128: return launch_bs<DT, 128>(prm, bs, stream);
    default: return hipErrorInvalidValue;
  }
}

size_t align256(size_t x) { return (x + 255) & ~(size_t)255; }

}  // namespace

AttnWorkspace attn_workspace_layout(int32_t num_seqs, int32_t slot_cols, int32_t num_q_heads,
                                    int32_t head_dim, int32_t max_context_len, int32_t stream_wgs) {
  AttnWorkspace ws{0, 0, 0, 0};
  if (num_seqs <= 0 || num_q_heads <= 0 || slot_cols <= 0 || head_dim <= 0) return ws;
  if (stream_wgs > 0) {
    // two piece slots per workgroup, then one parking row per wave
    const size_t slots = (size_t)stream_wgs * (2 + kWaves);
    ws.prefix_off = 0;
    ws.part_o_off = align256(sizeof(int32_t) * ((size_t)num_seqs + 1));
    ws.part_ml_off = align256(ws.part_o_off + slots * slot_cols * head_dim * sizeof(float));
    ws.bytes = ws.part_ml_off + slots * slot_cols * 2 * sizeof(float);
    return ws;
  }
  const int32_t P = max_context_len <= 0 ? 1
                                          : (max_context_len + kPartitionTokens - 1) / kPartitionTokens;
  if (P <= 1) return ws;
  const size_t rows = (size_t)num_seqs * num_q_heads * P;
  ws.part_o_off = 0;
  ws.part_ml_off = rows * head_dim * sizeof(float);
  ws.bytes = ws.part_ml_off + rows * 2 * sizeof(float);
  return ws;
}

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

hipError_t launch_paged_attention(const AttnParams& prm, int dtype, int head_dim,
                                  int block_size, hipStream_t stream) {
  switch (dtype) {
    case DT_F32: return launch_d<DT_F32>(prm, head_dim, block_size, stream);
    case DT_F16: return launch_d<DT_F16>(prm, head_dim, block_size, stream);
    case DT_BF16: return launch_d<DT_BF16>(prm, head_dim, block_size, stream);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace pkv
