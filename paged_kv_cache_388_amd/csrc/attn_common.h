// Device code shared by the decode kernels (attention.hip) and the prefill
// kernel (prefill.hip): vector types, the 16-token sub-tile loader, the
// matrix-core QK / online-softmax / PV core of one sub-tile, and the output
// helpers.  What each computes is described with the kernels that use it.
#pragma once

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
// Both patterns cover whole 128-byte lines per instruction.  K loaded
// straight in the MFMA operand layout instead (16 rows x 64 bytes per
// instruction, half lines: the KDIRECT variant of load_tile) gives the same
// decode time on the Llama-3-8B-shaped layer, but each line then takes two
// L2 requests (1.5x the requests in all); the whole-line loads and the LDS
// re-deal are kept.
template <int N>
struct Tile {
  uint4 k[N];
  uint32_t v[4][N];
};

// koff / voff: this lane's K / V byte offsets inside a 16-token sub-tile
// (the resources start at the sub-tile).  KDIRECT (a measurement variant):
// K is loaded straight in the MFMA A-operand order (lane l: token l & 15,
// 16-byte chunks (l >> 4) + 4 kk, koff = (l & 15) * row + 16 * (l >> 4)), so
// each instruction touches half lines and no LDS re-deal follows.
template <int N, bool KDIRECT = false>
__device__ __forceinline__ void load_tile(Tile<N>& t, rsrc_t kr, rsrc_t vr, int koff, int voff) {
  constexpr int kRow = 16 * 4 * N;  // bytes per token row = D * elem_bytes
  constexpr int kStep = KDIRECT ? 64 : 1024;
#pragma unroll
  for (int kk = 0; kk < N; ++kk)
    t.k[kk] = __builtin_bit_cast(
        uint4, __builtin_amdgcn_raw_buffer_load_b128(kr, koff + kk * kStep, 0, kStreamPolicy));
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

// attend_core for a sub-tile as loaded: K is re-dealt through `lds`, this
// wave's private staging slot (at least one sub-tile of K), unless it was
// loaded in the operand order already (KDIRECT).
template <int DT, int N, int kMM, bool KDIRECT = false>
__device__ __forceinline__ void attend_subtile(Tile<N>& t, const uint4 (&qb)[N], int valid,
                                               float scale_log2, int r, WaveState<kMM>& st,
                                               char* lds) {
  if constexpr (KDIRECT) {
    attend_core<DT, N, kMM>(t.k, t.v, qb, valid, scale_log2, r, st);
  } else {
    uint4 ka[N];
    restage_k<N>(ka, t, lds, threadIdx.x & 63);
    attend_core<DT, N, kMM>(ka, t.v, qb, valid, scale_log2, r, st);
  }
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

// Per-sequence column geometry, all wave-uniform.
struct SeqCols {
  int n;      // cached tokens
  int L;      // new tokens (query rows)
  int q0;     // first query row
  int ngrp;   // column groups
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

size_t align256(size_t x) { return (x + 255) & ~(size_t)255; }

// The clock builds' record: the real-time counter (100 MHz) at the start and
// at the end, the XCD the wave ran on (hardware register XCC_ID) in the low
// byte of word 2, and what the kernel adds to words 2 and 3.
__device__ __forceinline__ unsigned long long clock_now() { return __builtin_amdgcn_s_memrealtime(); }

__device__ __forceinline__ unsigned xcd_id() {
  unsigned x;
  asm volatile("s_getreg_b32 %0, hwreg(HW_REG_XCC_ID)" : "=s"(x));
  return x & 0xffu;
}

__device__ __forceinline__ void clock_record(unsigned long long* rec, long long index,
                                             unsigned long long t0, unsigned long long w2,
                                             unsigned long long w3) {
  if (index < 0 || index >= kClockRecords) return;
  unsigned long long* r = rec + index * kClockWords;
  r[0] = t0;
  r[1] = clock_now();
  r[2] = (unsigned long long)xcd_id() | (w2 << 8);
  r[3] = w3;
}

}  // namespace
}  // namespace pkv
