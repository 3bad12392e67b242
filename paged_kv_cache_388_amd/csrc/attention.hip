// Paged decode attention for gfx950 (CDNA4).
//
// What is computed: for each sequence s and query head h, attention of the
// single new query over the sequence's cached context, gathered through its
// block table (first page, "PagedAttention: Decoupling Logical Context from
// Contiguous GPU Memory"; "The Memory Wall", "Show Me The Code: A Conceptual
// PagedAttention Kernel", whose per-request loop over logical blocks with a
// table lookup per block is the structure kept here).  Query head h reads KV
// head h / G.
//
// Work decomposition.  One workgroup (4 waves) per (kv head, sequence,
// 512-token partition); all G query heads of the kv head share the K/V bytes
// it streams, so every K/V byte crosses HBM once per step.  Wave w takes the
// partition's 16-token sub-tiles w, w+4, w+8, ...
//
// Per 16-token sub-tile a wave does:
//   QK   S^T[16 tok x 16 cols] = K_tile[16 x D] . Q^T[D x 16] on MFMA
//        (16x16x32 for fp16/bf16, 16x16x4 for fp32).  Column g < G is query
//        head h*G+g; the other columns are zero padding.  Each lane's K load
//        is a 16-byte piece of one token row, which is exactly its A operand.
//   mask tokens at or past the context length get -inf (a select, so stale
//        or NaN bits in unused slots never reach the result).
//   softmax  running max per column (3 ops in-lane + 2 cross-row shuffles),
//        exp2 of base-2 logits, running normaliser, rescale of the
//        accumulator when the max grows.
//   PV   O^T[D x 16] += V^T[D x 16 tok] . P^T[16 tok x 16] on MFMA
//        (16x16x16).  P^T is the QK result already in place.  V^T is built
//        from natural 16-byte V loads: the head-dim index d is permuted so that
//        MFMA row rho, pass mm holds d = (D/16)*rho + mm, which makes each lane's
//        four token chunks the four k-values of its A operand (one v_perm_b32
//        per pair).  P is split into hi + lo 16-bit parts so the product keeps
//        ~16 mantissa bits instead of 8.
// The reduction order depends only on logical token positions.
//
// Partitions: a context longer than 512 tokens is split into 512-token
// partitions whose (max, normaliser, unnormalised output) are merged by a
// second kernel.  A single-partition context is finished in place.

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

constexpr int kWaves = 4;
constexpr int kThreads = 64 * kWaves;
constexpr int kSub = 16;  // tokens per MFMA row group
constexpr float kNegInf = -__builtin_huge_valf();

enum { DT_F32 = 0, DT_F16 = 1, DT_BF16 = 2 };

template <int DT> struct Elem { static constexpr int bytes = 2; };
template <> struct Elem<DT_F32> { static constexpr int bytes = 4; };

// Workgroups are dispatched round-robin over the 8 XCDs.  Remap the linear id
// so each XCD receives one contiguous range of the logical work order (kv
// head slowest): the sequences that read the same kv head's blocks, shared
// prefixes included, then meet in the same L2.
__device__ __forceinline__ int xcd_remap(int bid, int nblocks) {
  constexpr int kXcds = 8;
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

// One 16-token sub-tile in registers.  N = D * elem_bytes / 64.
//   k[kk]   : token (lane & 15), 16-byte chunk (lane >> 4) + 4*kk of its row
//   v[e][.] : token 4*(lane >> 4) + e, bytes [(lane & 15)*4N, +4N) of its row
template <int N>
struct Tile {
  uint4 k[N];
  uint32_t v[4][N];
};

template <int N>
__device__ __forceinline__ void load_tile(Tile<N>& t, const char* kbase, const char* vbase,
                                          int lane) {
  constexpr int kRow = 16 * 4 * N;  // bytes per token row = D * elem_bytes
  const int r = lane >> 4, c = lane & 15;
  const char* kp = kbase + c * kRow + r * 16;
#pragma unroll
  for (int kk = 0; kk < N; ++kk) t.k[kk] = *reinterpret_cast<const uint4*>(kp + kk * 64);
  const char* vp = vbase + (4 * r) * kRow + c * (4 * N);
#pragma unroll
  for (int e = 0; e < 4; ++e) {
    if constexpr (N == 2) {
      const uint2 x = *reinterpret_cast<const uint2*>(vp + e * kRow);
      t.v[e][0] = x.x; t.v[e][1] = x.y;
    } else {
#pragma unroll
      for (int j = 0; j < N / 4; ++j) {
        const uint4 x = *reinterpret_cast<const uint4*>(vp + e * kRow + 16 * j);
        t.v[e][4 * j + 0] = x.x; t.v[e][4 * j + 1] = x.y;
        t.v[e][4 * j + 2] = x.z; t.v[e][4 * j + 3] = x.w;
      }
    }
  }
}

template <int DT, int D, int BS>
__global__ __launch_bounds__(kThreads) void attn_partition_kernel(AttnParams prm) {
  constexpr int EB = Elem<DT>::bytes;
  constexpr int N = D * EB / 64;           // 16-byte K chunks per lane per sub-tile
  constexpr int kRow = D * EB;             // bytes per token row
  constexpr int kMM = D / 16;              // PV passes (MFMA row blocks of the head dim)
  static_assert(kPartitionTokens % BS == 0 && BS % kSub == 0, "partition/block sizes");

  __shared__ float sm_ml[kWaves][2][16];
  __shared__ float sm_o[kWaves][16][D + 4];

  const int lane = threadIdx.x & 63;
  const int w = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int r = lane >> 4;   // row group
  const int g = lane & 15;   // MFMA column = query head within the group

  const int P = prm.max_partitions;
  const int L = xcd_remap(blockIdx.x, gridDim.x);
  const int p = L % P;
  const int sh = L / P;
  const int s = sh % prm.num_seqs;
  const int h = sh / prm.num_seqs;
  const int G = prm.group;
  const int Hq = prm.num_q_heads;

  int ctx = prm.context_lens[s];
  ctx = ctx < 0 ? 0 : (ctx > prm.max_context_len ? prm.max_context_len : ctx);
  const int nparts = (ctx + kPartitionTokens - 1) / kPartitionTokens;
  if (p >= (nparts > 0 ? nparts : 1)) return;
  if (ctx == 0) {
    for (int idx = threadIdx.x; idx < G * D; idx += kThreads)
      store_out<DT>(prm.out, ((size_t)s * Hq + (size_t)h * G) * D + idx, 0.f);
    return;
  }

  const int tok0 = p * kPartitionTokens;
  const int ntok = min(kPartitionTokens, ctx - tok0);
  const int nsub = (ntok + kSub - 1) / kSub;
  const int niter = nsub > w ? (nsub - w + kWaves - 1) / kWaves : 0;

  // Block ids of this wave's sub-tiles: lane i holds the id for iteration i.
  const int32_t* bt_row = prm.block_tables + (size_t)s * prm.max_blocks_per_seq;
  int my_id = 0;
  if (lane < niter) my_id = bt_row[(tok0 + kSub * (w + kWaves * lane)) / BS];

  // Query operand (B of the QK MFMA): lane (r, g) holds query head h*G+g,
  // 16-byte chunks r + 4*kk of its row; zero for padding columns.
  uint4 qb[N];
  {
    const char* qrow = static_cast<const char*>(prm.q) +
                       (((size_t)s * Hq + (size_t)h * G + (g < G ? g : 0)) * D) * EB;
#pragma unroll
    for (int kk = 0; kk < N; ++kk) {
      qb[kk] = g < G ? *reinterpret_cast<const uint4*>(qrow + 16 * (r + 4 * kk))
                     : make_uint4(0, 0, 0, 0);
    }
  }

  const size_t tile_bytes = (size_t)BS * kRow;                 // one (block, head) tile
  const size_t block_bytes = tile_bytes * prm.num_kv_heads;
  const char* kpool = static_cast<const char*>(prm.k_cache) + (size_t)h * tile_bytes;
  const char* vpool = static_cast<const char*>(prm.v_cache) + (size_t)h * tile_bytes;
  const float scale_log2 = prm.scale_log2;

  float m_run = kNegInf;
  float l_run = 0.f;
  floatx4 acc[kMM];
#pragma unroll
  for (int mm = 0; mm < kMM; ++mm) acc[mm] = floatx4{0.f, 0.f, 0.f, 0.f};

  auto tile_ptrs = [&](int i, const char*& kb, const char*& vb) {
    int phys = __builtin_amdgcn_readlane(my_id, i);
    if ((unsigned)phys >= (unsigned)prm.num_blocks) phys = 0;  // never dereference a bad id
    const int off = (tok0 + kSub * (w + kWaves * i)) % BS;
    const size_t o = (size_t)phys * block_bytes + (size_t)off * kRow;
    kb = kpool + o;
    vb = vpool + o;
  };
  auto issue = [&](Tile<N>& t, int i) {
    const char *kb, *vb;
    tile_ptrs(i, kb, vb);
    load_tile<N>(t, kb, vb, lane);
  };
  auto compute = [&](Tile<N>& t, int i) {
    const int tokb = tok0 + kSub * (w + kWaves * i);
    const int phys = __builtin_amdgcn_readlane(my_id, i);
    int valid = ctx - tokb;
    valid = valid > kSub ? kSub : valid;
    if ((unsigned)phys >= (unsigned)prm.num_blocks) valid = 0;

    // ---- QK on MFMA --------------------------------------------------------
    floatx4 S = {0.f, 0.f, 0.f, 0.f};
    if constexpr (DT == DT_F32) {
#pragma unroll
      for (int kk = 0; kk < N; ++kk) {
        S = __builtin_amdgcn_mfma_f32_16x16x4f32(__uint_as_float(t.k[kk].x), __uint_as_float(qb[kk].x), S, 0, 0, 0);
        S = __builtin_amdgcn_mfma_f32_16x16x4f32(__uint_as_float(t.k[kk].y), __uint_as_float(qb[kk].y), S, 0, 0, 0);
        S = __builtin_amdgcn_mfma_f32_16x16x4f32(__uint_as_float(t.k[kk].z), __uint_as_float(qb[kk].z), S, 0, 0, 0);
        S = __builtin_amdgcn_mfma_f32_16x16x4f32(__uint_as_float(t.k[kk].w), __uint_as_float(qb[kk].w), S, 0, 0, 0);
      }
    } else if constexpr (DT == DT_F16) {
#pragma unroll
      for (int kk = 0; kk < N; ++kk)
        S = __builtin_amdgcn_mfma_f32_16x16x32_f16(__builtin_bit_cast(halfx8, t.k[kk]),
                                                   __builtin_bit_cast(halfx8, qb[kk]), S, 0, 0, 0);
    } else {
#pragma unroll
      for (int kk = 0; kk < N; ++kk)
        S = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, t.k[kk]),
                                                    __builtin_bit_cast(bf16x8, qb[kk]), S, 0, 0, 0);
    }

    // ---- mask + online softmax (lane (r, g) holds tokens 4r..4r+3 of column g)
    float sv[4];
#pragma unroll
    for (int e = 0; e < 4; ++e) sv[e] = (4 * r + e < valid) ? S[e] * scale_log2 : kNegInf;
    float mloc = fmaxf(fmaxf(sv[0], sv[1]), fmaxf(sv[2], sv[3]));
    mloc = fmaxf(mloc, __shfl_xor(mloc, 16));
    mloc = fmaxf(mloc, __shfl_xor(mloc, 32));
    const float m_new = fmaxf(m_run, mloc);
    const float mb = m_new == kNegInf ? 0.f : m_new;
    const float alpha = fast_exp2(m_run - mb);
    float pe[4];
#pragma unroll
    for (int e = 0; e < 4; ++e) pe[e] = fast_exp2(sv[e] - mb);
    l_run = l_run * alpha + ((pe[0] + pe[1]) + (pe[2] + pe[3]));
    m_run = m_new;
#pragma unroll
    for (int mm = 0; mm < kMM; ++mm) acc[mm] *= alpha;

    // ---- tail: V rows of masked tokens are zeroed (select, never 0 * v)
    if (valid < kSub) {
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const bool keep = 4 * r + e < valid;
#pragma unroll
        for (int j = 0; j < N; ++j) t.v[e][j] = keep ? t.v[e][j] : 0u;
      }
    }

    // ---- PV on MFMA ---------------------------------------------------------
    if constexpr (DT == DT_F32) {
#pragma unroll
      for (int mm = 0; mm < kMM; ++mm) {
#pragma unroll
        for (int e = 0; e < 4; ++e)
          acc[mm] = __builtin_amdgcn_mfma_f32_16x16x4f32(__uint_as_float(t.v[e][mm]), pe[e], acc[mm], 0, 0, 0);
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
        a.x = __builtin_amdgcn_perm(t.v[1][wd], t.v[0][wd], sel);
        a.y = __builtin_amdgcn_perm(t.v[3][wd], t.v[2][wd], sel);
        if constexpr (DT == DT_BF16) {
          const shortx4 A = __builtin_bit_cast(shortx4, a);
          acc[mm] = __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(A, __builtin_bit_cast(shortx4, phi),
                                                              acc[mm], 0, 0, 0);
          acc[mm] = __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(A, __builtin_bit_cast(shortx4, plo),
                                                              acc[mm], 0, 0, 0);
        } else {
          const halfx4 A = __builtin_bit_cast(halfx4, a);
          acc[mm] = __builtin_amdgcn_mfma_f32_16x16x16f16(A, __builtin_bit_cast(halfx4, phi),
                                                          acc[mm], 0, 0, 0);
          acc[mm] = __builtin_amdgcn_mfma_f32_16x16x16f16(A, __builtin_bit_cast(halfx4, plo),
                                                          acc[mm], 0, 0, 0);
        }
      }
    }
  };

  // Two register buffers: the next sub-tile's loads are in flight while the
  // current one is computed.  Loads are issued unconditionally (the index is
  // clamped to the last sub-tile) and the loop has a single exit, so the load
  // counter waits the compiler derives stay per-buffer instead of draining the
  // whole queue at the loop head.
  if (niter > 0) {
    Tile<N> ta, tb;
    issue(ta, 0);
    for (int i = 0; i + 1 < niter; i += 2) {
      issue(tb, i + 1);
      compute(ta, i);
      issue(ta, i + 2 < niter ? i + 2 : niter - 1);
      compute(tb, i + 1);
    }
    if (niter & 1) compute(ta, niter - 1);
  }

  // Column normaliser: sum over the four row groups.
  l_run += __shfl_xor(l_run, 16);
  l_run += __shfl_xor(l_run, 32);

  // ---- merge the four waves ------------------------------------------------
  if (g < G) {
    if (r == 0) {
      sm_ml[w][0][g] = m_run;
      sm_ml[w][1][g] = l_run;
    }
#pragma unroll
    for (int mm = 0; mm < kMM; ++mm) {
#pragma unroll
      for (int rr = 0; rr < 4; ++rr) sm_o[w][g][(D / 16) * (4 * r + rr) + mm] = acc[mm][rr];
    }
  }
  __syncthreads();

  for (int idx = threadIdx.x; idx < G * D; idx += kThreads) {
    const int gg = idx / D, d = idx % D;
    float M = kNegInf;
#pragma unroll
    for (int ww = 0; ww < kWaves; ++ww) M = fmaxf(M, sm_ml[ww][0][gg]);
    float lsum = 0.f, o = 0.f;
#pragma unroll
    for (int ww = 0; ww < kWaves; ++ww) {
      const float mw = sm_ml[ww][0][gg];
      const float f = mw == kNegInf ? 0.f : fast_exp2(mw - M);
      lsum += f * sm_ml[ww][1][gg];
      o += f * sm_o[ww][gg][d];
    }
    const size_t row = (size_t)s * Hq + (size_t)h * G + gg;
    if (nparts == 1) {
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
}

// Merge the partitions of one (sequence, query head): one wave, lanes over
// the head dim, partitions visited in logical order.
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
  for (int j = 0; j < kPer; ++j) store_out<DT>(prm.out, orow + lane + 64 * j, lsum > 0.f ? o[j] * inv : 0.f);
}

template <int DT, int D, int BS>
hipError_t launch_typed(const AttnParams& prm, hipStream_t stream) {
  const long long nwg = (long long)prm.num_seqs * prm.num_kv_heads * prm.max_partitions;
  if (nwg <= 0) return hipSuccess;
  if (nwg > 0x7fffffffLL) return hipErrorInvalidConfiguration;
  hipLaunchKernelGGL((attn_partition_kernel<DT, D, BS>), dim3((unsigned)nwg), dim3(kThreads), 0,
                     stream, prm);
  hipError_t err = hipGetLastError();
  if (err != hipSuccess || prm.max_partitions <= 1) return err;
  hipLaunchKernelGGL((attn_reduce_kernel<DT, D>), dim3((unsigned)(prm.num_seqs * prm.num_q_heads)),
                     dim3(64), 0, stream, prm);
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

}  // namespace

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
