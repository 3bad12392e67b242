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


#include "attn_common.h"

namespace pkv {
namespace {

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

// Tokens of sub-tile t that column group cg can see at all (its last
// column's causal limit), 0..16: later rows are not loaded.
__device__ __forceinline__ int group_rows(const SeqCols& sc, int cg, int G, int t) {
  int i_last = (cg * kSub + kSub - 1) / G;
  i_last = i_last < sc.L - 1 ? i_last : sc.L - 1;
  int v = sc.n - sc.L + i_last + 1 - t * kSub;
  return v > kSub ? kSub : v;
}

// kClock: the measurement build, which also records each wave's start and
// end (see clock_record; word 2 adds the wave's positions and the pieces it
// finished, word 3 its workgroup as numbered by xcd_remap).
template <int DT, int D, int BS, bool MULTI, bool KDIRECT = false, bool kClock = false>
__global__ __launch_bounds__(kThreads) __attribute__((amdgpu_waves_per_eu(2)))
void attn_stream_kernel(AttnParams prm) {
  [[maybe_unused]] unsigned long long clk0 = 0;
  [[maybe_unused]] int clk_pieces = 0;
  if constexpr (kClock) clk0 = clock_now();
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

  const int koff = KDIRECT ? (lane & 15) * Geo::kRow + 16 * r : 16 * lane;
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
      load_tile<N, KDIRECT>(t, make_rsrc(static_cast<const char*>(prm.k_cache) + sub, nrec),
                            make_rsrc(static_cast<const char*>(prm.v_cache) + sub, nrec), koff,
                            voff);
      ++pi;
      if (pi < b && pi == si.E) enter_issue_seq();
    } else {
      // past the chunk: keep the per-slot load count fixed, touch no memory
      m.p = -1;
      load_tile<N, KDIRECT>(t, make_rsrc(prm.k_cache, 0), make_rsrc(prm.v_cache, 0), koff, voff);
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
    attend_subtile<DT, N, kMM, KDIRECT>(t, qb, valid, scale_log2, r, st, kst);
    if (m.p + 1 == sc.E || m.p + 1 == b) {
      if constexpr (kClock) ++clk_pieces;
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
  if constexpr (kClock)
    if (lane == 0)
      clock_record(prm.clock, wv, clk0, (unsigned long long)(b - a) | ((unsigned long long)clk_pieces << 32),
                   (unsigned long long)wg);
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

template <int DT, int D, int BS>
hipError_t launch_typed(const AttnParams& prm, hipStream_t stream) {
  const dim3 block(kThreads);
  const long long nout = (long long)prm.num_seqs * prm.num_q_heads;
  if (nout > 0x7fffffffLL) return hipErrorInvalidConfiguration;
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
    // K loaded straight in the MFMA operand order, and the clock build: two
    // measurement variants, built for one shape only (bf16, D 128, 16-token
    // blocks)
    constexpr bool kDirectBuilt = DT == DT_BF16 && D == 128 && BS == 16;
    if (prm.clock && kDirectBuilt)
      hipLaunchKernelGGL((attn_stream_kernel<DT, D, BS, false, false, kDirectBuilt>),
                         dim3((unsigned)prm.stream_wgs), block, 0, stream, prm);
    else if (prm.k_direct && kDirectBuilt)
      hipLaunchKernelGGL((attn_stream_kernel<DT, D, BS, false, kDirectBuilt>),
                         dim3((unsigned)prm.stream_wgs), block, 0, stream, prm);
    else
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

hipError_t launch_paged_attention(const AttnParams& prm, int dtype, int head_dim,
                                  int block_size, hipStream_t stream) {
  if (prm.prefill_blocks > 0) return launch_prefill(prm, dtype, head_dim, block_size, stream);
  switch (dtype) {
    case DT_F32: return launch_d<DT_F32>(prm, head_dim, block_size, stream);
    case DT_F16: return launch_d<DT_F16>(prm, head_dim, block_size, stream);
    case DT_BF16: return launch_d<DT_BF16>(prm, head_dim, block_size, stream);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace pkv
