// Router and alignment kernels of the MoE-LoRA layer (gfx950).
//
// The alignment groups the routed rows per expert, pads each group to the
// shared block size BM, and orders each group by adapter (base-only rows
// last) and then by row index.  It is the structure that lets one grouped
// GEMM serve expert routing and adapter selection at once: the AWS ML blog
// "Efficiently serve dozens of fine-tuned models with vLLM on Amazon
// SageMaker AI and Amazon Bedrock", section "Implementing multi-LoRA
// inference for MoE models in vLLM" (compound sparsity of expert routing and
// adapter selection), and section "Tuning kernel configurations for Amazon
// SageMaker AI and Amazon Bedrock" (one BLOCK_SIZE_M shared by the four LoRA
// ops).  Every output is a pure function of the ids, so it is reproducible
// bit for bit: counts come from integer atomics and every position from
// stable ranks, never from the order in which atomics happen to land.
#include "common.h"
#include "kernels.h"
#include "rowlora.h"

#include <type_traits>

namespace moelora {

namespace {

constexpr int kAlignThreads = 1024;
constexpr int kAlignWaves = kAlignThreads / kWave;
constexpr int kMaxBuckets = 8448;   // E * (NA + 1)
constexpr int kMaxAdapterRanks = 256;  // NA + 1
constexpr int kScatterThreads = 512;

__device__ __forceinline__ unsigned long long lanemask_lt(int lane) {
  return (1ull << lane) - 1ull;
}

// DPP controls (gfx9): quad permutations, row shifts, half-row and row
// mirrors, broadcasts of a row's last lane into the rows above
constexpr int kDppQuadSwap1 = 0xb1;  // quad_perm [1, 0, 3, 2]
constexpr int kDppQuadSwap2 = 0x4e;  // quad_perm [2, 3, 0, 1]
constexpr int kDppHalfMirror = 0x141;
constexpr int kDppMirror = 0x140;
constexpr int kDppRowShr = 0x110;  // + shift (1..15)
constexpr int kDppBcast15 = 0x142, kDppBcast31 = 0x143;
__device__ __forceinline__ unsigned dpp_max(unsigned x, unsigned y) { return x > y ? x : y; }
template <int CTRL>
__device__ __forceinline__ unsigned dpp_mov(unsigned x) {
  return (unsigned)__builtin_amdgcn_update_dpp(0, (int)x, CTRL, 0xf, 0xf, false);
}
// Inclusive prefix sum over the 64 lanes of a wave (every lane active), by
// DPP: shifts by 1, 2, 4, 8 inside each 16-lane row (lanes shifted in from
// outside the row read 0), then row 15's total added into rows 1 and 3 and
// lane 31's into rows 2 and 3 -- six moves where lane shuffles pay an
// LDS-crossbar round trip per step.
__device__ __forceinline__ int wave_incl_scan(int x) {
  x += __builtin_amdgcn_update_dpp(0, x, kDppRowShr + 1, 0xf, 0xf, false);
  x += __builtin_amdgcn_update_dpp(0, x, kDppRowShr + 2, 0xf, 0xf, false);
  x += __builtin_amdgcn_update_dpp(0, x, kDppRowShr + 4, 0xf, 0xf, false);
  x += __builtin_amdgcn_update_dpp(0, x, kDppRowShr + 8, 0xf, 0xf, false);
  x += __builtin_amdgcn_update_dpp(0, x, kDppBcast15, 0xa, 0xf, false);
  x += __builtin_amdgcn_update_dpp(0, x, kDppBcast31, 0xc, 0xf, false);
  return x;
}

// Exclusive prefix sum over the 1024 threads of the block; *total gets the
// sum.  tmp holds kAlignWaves ints.  Contains two barriers.
__device__ int block_excl_scan(int v, int *tmp, int *total) {
  const int lane = threadIdx.x & (kWave - 1), w = threadIdx.x / kWave;
  const int x = wave_incl_scan(v);
  if (lane == kWave - 1) tmp[w] = x;
  __syncthreads();
  int off = 0, tot = 0;
#pragma unroll
  for (int i = 0; i < kAlignWaves; ++i) {
    int t = tmp[i];
    off += (i < w) ? t : 0;
    tot += t;
  }
  __syncthreads();
  *total = tot;
  return off + x - v;
}

// block_excl_scan of two values at once (same two barriers).
__device__ int2 block_excl_scan2(int v0, int v1, int2 *tmp, int2 *total) {
  const int lane = threadIdx.x & (kWave - 1), w = threadIdx.x / kWave;
  const int x0 = wave_incl_scan(v0), x1 = wave_incl_scan(v1);
  if (lane == kWave - 1) tmp[w] = make_int2(x0, x1);
  __syncthreads();
  int2 off = make_int2(0, 0), tot = make_int2(0, 0);
#pragma unroll
  for (int i = 0; i < kAlignWaves; ++i) {
    const int2 u = tmp[i];
    if (i < w) {
      off.x += u.x;
      off.y += u.y;
    }
    tot.x += u.x;
    tot.y += u.y;
  }
  __syncthreads();
  *total = tot;
  return make_int2(off.x + x0 - v0, off.y + x1 - v1);
}

// Router for one token, computed by one wave: the k largest logits (ties to
// the lower expert index, largest first) and their softmax over the kept
// logits.  Lane l holds experts l, l + 64, ...; each of the k rounds finds
// the largest untaken logit and then, by ballots in expert order, the lowest
// expert index holding it.  The maximum is taken on order-preserving
// unsigned images of the floats (sign bit flipped for non-negative values,
// every bit for negative ones; -0 taken as +0, which compares equal to it,
// and every image at least 1, so 0 marks an absent or taken expert): DPP moves inside each 16-lane row (quad
// swaps, then the half-row and row mirrors), then the four row maxima read
// into scalars -- a few cycles per step where a butterfly of lane shuffles
// pays an LDS-crossbar round trip per step.  Lanes j < k end with the j-th
// pick in (*id, *wt).
// SLOTS = experts per lane (E <= 64 * SLOTS), a template so that small
// expert counts run a short serial path.
__device__ __forceinline__ unsigned float_order_key(float f) {
  unsigned u = __float_as_uint(f);
  if ((u << 1) == 0u) u = 0u;  // -0 -> +0
  const unsigned key = (u & 0x80000000u) ? ~u : (u | 0x80000000u);
  return key > 1u ? key : 1u;  // only a negative NaN's image could be 0
}
__device__ __forceinline__ float float_of_order_key(unsigned k) {
  return __uint_as_float((k & 0x80000000u) ? (k & 0x7fffffffu) : ~k);
}
// the wave-wide maximum, in every lane (scalar)
__device__ __forceinline__ unsigned wave_max_u32(unsigned x) {
  x = dpp_max(x, dpp_mov<kDppQuadSwap1>(x));
  x = dpp_max(x, dpp_mov<kDppQuadSwap2>(x));
  x = dpp_max(x, dpp_mov<kDppHalfMirror>(x));  // lane i meets 7 - i: max of 8
  x = dpp_max(x, dpp_mov<kDppMirror>(x));      // lane i meets 15 - i: max of 16
  const unsigned r0 = __builtin_amdgcn_readlane(x, 0), r1 = __builtin_amdgcn_readlane(x, 16);
  const unsigned r2 = __builtin_amdgcn_readlane(x, 32), r3 = __builtin_amdgcn_readlane(x, 48);
  return dpp_max(dpp_max(r0, r1), dpp_max(r2, r3));
}

template <int SLOTS>
__device__ void route_token_rounds(const float *__restrict__ row, int E, int k, int *id, float *wt) {
  const int lane = threadIdx.x & (kWave - 1);
  unsigned key[SLOTS];  // 0 for an absent or taken expert (below every logit's image)
#pragma unroll
  for (int i = 0; i < SLOTS; ++i) {
    const int e = lane + i * kWave;
    key[i] = e < E ? float_order_key(row[e]) : 0u;
  }
  float my_val = 0.f, top = 0.f;
  int my_id = 0;
  for (int j = 0; j < k; ++j) {
    unsigned m = 0;
#pragma unroll
    for (int i = 0; i < SLOTS; ++i) m = dpp_max(m, key[i]);
    m = wave_max_u32(m);
    int bi = 0;
#pragma unroll
    for (int i = SLOTS - 1; i >= 0; --i) {  // the lowest slot holding m wins
      const unsigned long long b = __ballot(key[i] == m);
      if (b) bi = i * kWave + __ffsll((long long)b) - 1;
    }
    if ((bi & (kWave - 1)) == lane) {
#pragma unroll
      for (int i = 0; i < SLOTS; ++i)
        if (i == bi / kWave) key[i] = 0u;
    }
    const float bv = float_of_order_key(m);
    if (j == 0) top = bv;
    if (lane == j) {
      my_val = bv;
      my_id = bi;
    }
  }
  const float ex = lane < k ? expf(my_val - top) : 0.f;
  float sum = ex;
#pragma unroll
  for (int d = kWave / 2; d >= 1; d >>= 1) sum += __shfl_xor(sum, d);
  *id = my_id;
  *wt = ex / sum;
}

// The same router by ranks, for up to 64 experts: expert e's rank is the
// number of experts that beat it (a larger logit, or an equal one at a lower
// index), so for finite logits the ranks are a permutation and the picks are
// the ranks 0 .. k-1, in the same order as the rounds above.  Each lane
// counts for its experts against every logit of the row, broadcast from the
// lane holding it; the picks come out with ballots and lane reads, and the
// renormalising sum runs in pick order.
template <int SLOTS>
__device__ void route_token_ranked(const float *__restrict__ row, int E, int k, int *id, float *wt) {
  const int lane = threadIdx.x & (kWave - 1);
  float v[SLOTS];
  int rank[SLOTS];
#pragma unroll
  for (int i = 0; i < SLOTS; ++i) {
    const int e = lane + i * kWave;
    v[i] = e < E ? row[e] : 0.f;
    rank[i] = e < E ? 0 : E;  // absent experts are never picked
  }
#pragma unroll
  for (int s = 0; s < SLOTS; ++s) {
    const int n = min(kWave, E - s * kWave);
    for (int l = 0; l < n; ++l) {
      const int q = l + s * kWave;
      const float u = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v[s]), l));
#pragma unroll
      for (int i = 0; i < SLOTS; ++i)
        rank[i] += (u > v[i] || (u == v[i] && q < lane + i * kWave)) ? 1 : 0;
    }
  }
  float top = 0.f, sum = 0.f, my_ex = 0.f;
  int my_id = 0;
  for (int j = 0; j < k; ++j) {
    int ej = 0;  // a non-finite logit can leave a rank unfilled: expert 0 then
    float vj = 0.f;
#pragma unroll
    for (int i = 0; i < SLOTS; ++i) {
      const unsigned long long b = __ballot(rank[i] == j);
      if (b) {
        const int l = __ffsll((long long)b) - 1;
        ej = l + i * kWave;
        vj = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v[i]), l));
      }
    }
    if (j == 0) top = vj;
    const float ex = expf(vj - top);
    sum += ex;
    if (lane == j) {
      my_id = ej;
      my_ex = ex;
    }
  }
  *id = my_id;
  *wt = my_ex / sum;
}

template <int SLOTS>
__device__ void route_token(const float *__restrict__ row, int E, int k, int *id, float *wt) {
  // ranks measured faster up to 64 experts (the routing + alignment launch
  // of 64 tokens over 8 experts: 24.5 -> 20.7 us); at 128 experts the E
  // broadcasts per lane cost more than the rounds
  if constexpr (SLOTS == 1)
    route_token_ranked<SLOTS>(row, E, k, id, wt);
  else
    route_token_rounds<SLOTS>(row, E, k, id, wt);
}

// One wave per token.
template <int SLOTS>
__global__ __launch_bounds__(256) void k_route(const float *__restrict__ logits, int T, int E,
                                               int k, int *__restrict__ ids,
                                               float *__restrict__ w) {
  const int lane = threadIdx.x & (kWave - 1);
  const int t = blockIdx.x * (blockDim.x / kWave) + threadIdx.x / kWave;
  if (t >= T) return;
  int id;
  float wt;
  route_token<SLOTS>(logits + (size_t)t * E, E, k, &id, &wt);
  if (lane < k) {
    ids[(size_t)t * k + lane] = id;
    w[(size_t)t * k + lane] = wt;
  }
}

// The block size BM is a power of two (16, 32, 64 or 128 rows), so block
// indices of positions are shifts: a division by a runtime value costs ~35
// VALU instructions, and the plan and store loops below take one per bucket
// and per (block, adapter), over thousands of buckets (in the 128-expert,
// 32-adapter layer they were 14 of the one-workgroup kernel's 21 us).
__device__ __forceinline__ int log2_bm(int BM) { return 31 - __builtin_clz(BM); }
// blocks covered by the c >= 1 positions starting at st
__device__ __forceinline__ int blocks_spanned(int st, int c, int lb) {
  return ((st + c - 1) >> lb) - (st >> lb) + 1;
}

__device__ __forceinline__ int adapter_rank(const int *aid, int t, int NA, int &err) {
  if (!aid) return NA;
  const int a = aid[t];
  if (a < -1 || a >= NA) err |= MOELORA_DEVERR_ADAPTER_ID;
  return (a >= 0 && a < NA) ? a : NA;
}

constexpr int kMaxExperts = 1024;
// buckets per thread in align_plan / align_store (consecutive buckets)
constexpr int kBucketChunk = (kMaxBuckets + kAlignThreads - 1) / kAlignThreads;

struct AlignSmem {
  int hist[kMaxBuckets];      // rows per (expert, adapter rank) bucket; after align_plan its start
  int seg0[kMaxExperts + 1];  // padded expert segment starts, seg0[E] = padded total
  int rows[kMaxExperts];      // routed rows per expert
  int p0[kMaxExperts];        // rows of the experts before e (unpadded)
  int tile0[kMaxExperts];     // index of expert e's first LoRA tile
  int scan_tmp[kAlignWaves];
  int2 scan_tmp2[kAlignWaves];
  int totals[3];              // align_plan_wave: padded rows, LoRA segments, tiles
};

// Everything that follows from the bucket histogram (in LDS): padded expert
// segments, bucket start positions, padding sentinels, block experts, LoRA
// segments and their block tiles, the first tile of every block, and the
// counts.  Thread i takes the consecutive buckets [b0, b0 + nb) (bucket
// order is (expert, adapter rank)), so the LoRA segment and tile lists, which
// follow bucket order, come out of three block-wide scans with no serial
// loop over an expert's buckets; a block finds its expert by binary search
// over the segment starts.
//
// Two phases, because a workgroup barrier waits for every global store the
// workgroup has in flight: align_plan runs the scans (barriers, LDS only)
// and turns sm.hist[b] into the start position of bucket b; align_store
// then issues every global store with no barrier after it.
struct AlignPlan {
  int c[kBucketChunk];        // row counts of the thread's buckets
  int b0, nb;                 // the thread's buckets
  int seg_off, tile_off;      // first LoRA segment / tile of the thread's buckets
  int num_padded, n_seg, n_tiles;
};

__device__ AlignPlan align_plan(const Shape &s, AlignSmem &sm) {
  const int tid = threadIdx.x;
  const int E = s.E, NA = s.NA, NR = NA + 1, BM = s.BM, NB = E * NR;
  int *hist = sm.hist;
  AlignPlan P{};
  const int per = (NB + kAlignThreads - 1) / kAlignThreads;
  P.b0 = min(tid * per, NB);
  P.nb = min(per, NB - P.b0);
  int sum = 0;
#pragma unroll
  for (int i = 0; i < kBucketChunk; ++i) {
    P.c[i] = i < P.nb ? hist[P.b0 + i] : 0;
    sum += P.c[i];
  }
  // unpadded start of every bucket (its counts are read: the scan's barriers
  // order the overwrite after every thread's read)
  int total;
  int run = block_excl_scan(sum, sm.scan_tmp, &total);
#pragma unroll
  for (int i = 0; i < kBucketChunk; ++i)
    if (i < P.nb) {
      hist[P.b0 + i] = run;
      run += P.c[i];
    }
  __syncthreads();
  // experts: routed rows, padded segment starts
  const bool owner = tid < E;  // E <= 1024: one expert per thread
  int rows = 0, pstart = 0;
  if (owner) {
    pstart = hist[tid * NR];
    rows = (tid + 1 < E ? hist[(tid + 1) * NR] : total) - pstart;
  }
  const int lb = log2_bm(BM);
  const int padded = ((rows + BM - 1) >> lb) << lb;
  int np;
  const int seg0 = block_excl_scan(padded, sm.scan_tmp, &np);
  if (owner) {
    sm.seg0[tid] = seg0;
    sm.rows[tid] = rows;
    sm.p0[tid] = pstart;
    if (tid == E - 1) sm.seg0[E] = np;
  }
  __syncthreads();
  // padded bucket starts; LoRA segments and block tiles of the thread's buckets
  int nseg = 0, ntile = 0;
  const int e0 = P.b0 / NR, a0 = P.b0 - e0 * NR;  // (expert, rank) of the first bucket
  {
    int e = e0, a = a0;
#pragma unroll
    for (int i = 0; i < kBucketChunk; ++i) {
      if (i < P.nb) {
        const int b = P.b0 + i;
        const int st = sm.seg0[e] + hist[b] - sm.p0[e];
        hist[b] = st;
        if (a < NA && P.c[i] > 0) {
          ++nseg;
          ntile += blocks_spanned(st, P.c[i], lb);
        }
      }
      if (++a == NR) {
        a = 0;
        ++e;
      }
    }
  }
  int2 tot;
  const int2 off = block_excl_scan2(nseg, ntile, sm.scan_tmp2, &tot);
  // each expert's first tile index, from the thread holding its first bucket
  int ti = off.y;
  {
    int e = e0, a = a0;
#pragma unroll
    for (int i = 0; i < kBucketChunk; ++i) {
      if (i < P.nb) {
        const int b = P.b0 + i;
        if (a == 0) sm.tile0[e] = ti;
        if (a < NA && P.c[i] > 0) ti += blocks_spanned(hist[b], P.c[i], lb);
      }
      if (++a == NR) {
        a = 0;
        ++e;
      }
    }
  }
  __syncthreads();
  P.seg_off = off.x;
  P.tile_off = off.y;
  P.n_seg = tot.x;
  P.n_tiles = tot.y;
  P.num_padded = np;
  return P;
}

// Exclusive prefix sum over the 64 lanes of a wave; *total gets the sum.
__device__ __forceinline__ int wave_excl_scan(int v, int *total) {
  const int x = wave_incl_scan(v);
  *total = __builtin_amdgcn_readlane(x, kWave - 1);
  return x - v;
}

// align_plan for few experts and buckets (E <= 64, E (NA + 1) <= 64
// kBucketChunk): wave 0 alone runs the same three scans at wave level, so
// the plan has one workgroup barrier instead of eight (a decode step's
// 288 buckets: ~5 us of block scans otherwise).  Same results.
__device__ __forceinline__ bool align_plan_wave_ok(const Shape &s) {
  return s.E <= kWave && s.E * (s.NA + 1) <= kWave * kBucketChunk;
}

__device__ AlignPlan align_plan_wave(const Shape &s, AlignSmem &sm) {
  const int tid = threadIdx.x;
  const int E = s.E, NA = s.NA, NR = NA + 1, BM = s.BM, NB = E * NR;
  int *hist = sm.hist;
  AlignPlan P{};
  if (tid < kWave) {
    const int per = (NB + kWave - 1) / kWave;
    P.b0 = min(tid * per, NB);
    P.nb = min(per, NB - P.b0);
    int sum = 0;
#pragma unroll
    for (int i = 0; i < kBucketChunk; ++i) {
      P.c[i] = i < P.nb ? hist[P.b0 + i] : 0;
      sum += P.c[i];
    }
    int total;
    int run = wave_excl_scan(sum, &total);
    // (a wave's LDS accesses complete in program order)
#pragma unroll
    for (int i = 0; i < kBucketChunk; ++i)
      if (i < P.nb) {
        hist[P.b0 + i] = run;
        run += P.c[i];
      }
    int rows = 0, pstart = 0;
    if (tid < E) {
      pstart = hist[tid * NR];
      rows = (tid + 1 < E ? hist[(tid + 1) * NR] : total) - pstart;
    }
    const int lb = log2_bm(BM);
    const int padded = ((rows + BM - 1) >> lb) << lb;
    int np;
    const int seg0 = wave_excl_scan(padded, &np);
    if (tid < E) {
      sm.seg0[tid] = seg0;
      sm.rows[tid] = rows;
      sm.p0[tid] = pstart;
    }
    if (tid == 0) sm.seg0[E] = np;
    int nseg = 0, ntile = 0;
    const int e0 = P.b0 / NR, a0 = P.b0 - e0 * NR;
    {
      int e = e0, a = a0;
#pragma unroll
      for (int i = 0; i < kBucketChunk; ++i) {
        if (i < P.nb) {
          const int b = P.b0 + i;
          const int st = sm.seg0[e] + hist[b] - sm.p0[e];
          hist[b] = st;
          if (a < NA && P.c[i] > 0) {
            ++nseg;
            ntile += blocks_spanned(st, P.c[i], lb);
          }
        }
        if (++a == NR) {
          a = 0;
          ++e;
        }
      }
    }
    int n_seg, n_tiles;
    P.seg_off = wave_excl_scan(nseg, &n_seg);
    P.tile_off = wave_excl_scan(ntile, &n_tiles);
    int ti = P.tile_off;
    {
      int e = e0, a = a0;
#pragma unroll
      for (int i = 0; i < kBucketChunk; ++i) {
        if (i < P.nb) {
          const int b = P.b0 + i;
          if (a == 0) sm.tile0[e] = ti;
          if (a < NA && P.c[i] > 0) ti += blocks_spanned(hist[b], P.c[i], lb);
        }
        if (++a == NR) {
          a = 0;
          ++e;
        }
      }
    }
    if (tid == 0) {
      sm.totals[0] = np;
      sm.totals[1] = n_seg;
      sm.totals[2] = n_tiles;
    }
  }
  __syncthreads();
  P.num_padded = sm.totals[0];
  P.n_seg = sm.totals[1];
  P.n_tiles = sm.totals[2];
  return P;
}

__device__ void align_store(const Shape &s, const AlignSmem &sm, const AlignPlan &P,
                            const AlignBufs &al) {
  const int tid = threadIdx.x;
  const int E = s.E, NA = s.NA, NR = NA + 1, BM = s.BM, R = s.R;
  const int *start = sm.hist;
  const int np = P.num_padded;
  const int lb = log2_bm(BM);
  // the thread's buckets: start and row count, LoRA segment and block tiles
  int si = P.seg_off, ti = P.tile_off;
  int be = P.b0 / NR, ba = P.b0 - be * NR;  // (expert, rank) of bucket b0 + i
#pragma unroll
  for (int i = 0; i < kBucketChunk; ++i) {
    if (i < P.nb) {
      const int b = P.b0 + i;
      const int st = start[b], c = P.c[i];
      al.bucket_base[b] = st;
      al.bucket_cnt[b] = c;
      if (ba < NA && c > 0) {
        reinterpret_cast<int4 *>(al.lora_seg)[si++] = make_int4(be, ba, st, c);
        for (int blk = st >> lb; blk <= (st + c - 1) >> lb; ++blk) {
          const int lo = max(st, blk << lb), hi = min(st + c, (blk + 1) << lb);
          if (lo == blk << lb) al.block_tile_start[blk] = ti;  // the block's first tile
          reinterpret_cast<int4 *>(al.tiles)[ti++] = make_int4(blk, ba, lo - (blk << lb), hi - lo);
        }
      }
    }
    if (++ba == NR) {
      ba = 0;
      ++be;
    }
  }
  // blocks: expert (the last one whose segment starts at or before the
  // block; empty experts share their start with the next) and first tile.
  // An expert's rows with an adapter come first, so a block has LoRA tiles
  // exactly when its first position holds such a row, and then its first
  // tile starts at the block start (written with the tiles above); any
  // other block of expert e comes after all of e's tiles: its first tile is
  // the next expert's first tile.
  for (int b = tid; b < s.nblk; b += kAlignThreads) {
    int e = -1, t = P.n_tiles;
    bool tiled = false;
    if (b < (np >> lb)) {
      const int pos = b << lb;
      int lo = 0, hi = E;
      while (hi - lo > 1) {
        const int mid = (lo + hi) >> 1;
        if (sm.seg0[mid] <= pos) lo = mid; else hi = mid;
      }
      e = lo;
      tiled = pos < start[e * NR + NA];  // the start of e's rows without an adapter
      if (!tiled && e + 1 < E) t = sm.tile0[e + 1];
    }
    al.block_expert[b] = e;
    if (!tiled) al.block_tile_start[b] = t;
  }
  if (tid < E) al.seg_start[tid] = sm.seg0[tid];
  // padding sentinels: slot j < BM - 1 past the end of each expert's rows
  for (int i = tid; i < (E << lb); i += kAlignThreads) {
    const int e = i >> lb, j = i & (BM - 1);
    const int pos = sm.seg0[e] + sm.rows[e] + j;
    if (j < BM - 1 && pos < sm.seg0[e + 1]) al.sorted_rows[pos] = R;
  }
  if (tid == 0) {
    al.seg_start[E] = np;
    al.block_tile_start[s.nblk] = P.n_tiles;
    al.counts[0] = np;
    al.counts[1] = P.n_seg;
    al.counts[2] = P.n_tiles;
    al.counts[3] = 0;
  }
  for (int i = np + tid; i < s.cap; i += kAlignThreads) al.sorted_rows[i] = R;
  for (int i = P.n_seg + tid; i < s.max_seg; i += kAlignThreads)
    reinterpret_cast<int4 *>(al.lora_seg)[i] = make_int4(-1, -1, 0, 0);
  for (int i = P.n_tiles + tid; i < s.max_tiles; i += kAlignThreads)
    reinterpret_cast<int4 *>(al.tiles)[i] = make_int4(-1, -1, 0, 0);
}

// Alignment metadata for any batch, one workgroup: bucket histogram, then
// align_layout, then the tokens ordered by adapter rank (for the scatter).
__global__ __launch_bounds__(kAlignThreads) void k_align_meta(Shape s, const int *__restrict__ ids,
                                                              const int *__restrict__ aid,
                                                              AlignBufs al) {
  __shared__ AlignSmem sm;
  __shared__ int tok_cnt[kMaxAdapterRanks];
  __shared__ int tok_base[kMaxAdapterRanks];
  __shared__ int cursor[kMaxAdapterRanks];
  __shared__ int wtab[kAlignWaves][kMaxAdapterRanks];
  __shared__ int err_all;

  const int tid = threadIdx.x, lane = tid & (kWave - 1), wv = tid / kWave;
  const int E = s.E, NA = s.NA, NR = NA + 1, R = s.R, k = s.k, T = s.T;
  const int NB = E * NR;

  for (int i = tid; i < NB; i += kAlignThreads) sm.hist[i] = 0;
  for (int i = tid; i < NR; i += kAlignThreads) {
    tok_cnt[i] = 0;
    cursor[i] = 0;
  }
  for (int i = tid; i < kAlignWaves * NR; i += kAlignThreads) wtab[i / NR][i % NR] = 0;
  if (tid == 0) err_all = 0;
  __syncthreads();

  // Tokens per adapter rank and rows per (expert, adapter rank) bucket.
  // Each pass takes up to kHistBatch tokens and kRowBatch rows per thread
  // and issues all their loads (clamped indices) before the first use, so a
  // pass pays the global load latency once; the LDS atomics follow.  Slots
  // past the end for the whole workgroup are skipped by uniform branches
  // (one workgroup retires about one wave instruction per clock, so dead
  // slots cost time).
  // Tokens per adapter rank: a wave adds each of its distinct ranks once
  // (a prefill's tokens share a few adapters, and per-lane atomics on one
  // LDS word serialize).
  // A row's token p / k by a multiply-high: with m = ceil(2^32 / k) the
  // product's high word is exact while p k < 2^32 (the error p (m - 2^32 / k)
  // / 2^32 stays below 1 / k).
  constexpr int kHistBatch = 8, kRowBatch = 16;
  const bool magic_ok = k > 1 && (unsigned long long)R * (unsigned)k < (1ull << 32);
  const unsigned kmagic = magic_ok ? (unsigned)(((1ull << 32) + k - 1) / k) : 0u;
  const int npass = max((T + kHistBatch * kAlignThreads - 1) / (kHistBatch * kAlignThreads),
                        (R + kRowBatch * kAlignThreads - 1) / (kRowBatch * kAlignThreads));
  int err = 0;
  for (int pass = 0; pass < npass; ++pass) {
    const int t0 = tid + pass * kHistBatch * kAlignThreads;
    const int p0 = tid + pass * kRowBatch * kAlignThreads;
    // live slots (uniform): slot u has a token / row for some thread
    const int nt = min(kHistBatch, max(0, T - pass * kHistBatch * kAlignThreads + kAlignThreads - 1) /
                                           kAlignThreads);
    const int nr = min(kRowBatch, max(0, R - pass * kRowBatch * kAlignThreads + kAlignThreads - 1) /
                                          kAlignThreads);
    int ta[kHistBatch], re[kRowBatch], ra[kRowBatch];
#pragma unroll
    for (int u = 0; u < kHistBatch; ++u)
      ta[u] = (u < nt && aid) ? aid[min(t0 + u * kAlignThreads, T - 1)] : -1;
#pragma unroll
    for (int u = 0; u < kRowBatch; ++u) {
      re[u] = ra[u] = -1;
      if (u >= nr) continue;
      const int p = min(p0 + u * kAlignThreads, R - 1);
      const int t = k == 1 ? p : magic_ok ? (int)__umulhi((unsigned)p, kmagic) : p / k;
      re[u] = ids[p];
      ra[u] = aid ? aid[t] : -1;
    }
#pragma unroll
    for (int u = 0; u < kHistBatch; ++u) {
      if (u >= nt) break;
      const int a = ta[u];
      const bool live = t0 + u * kAlignThreads < T;
      if (live && (a < -1 || a >= NA)) err |= MOELORA_DEVERR_ADAPTER_ID;
      const int ar = !live ? -1 : (a >= 0 && a < NA) ? a : NA;
      unsigned long long active = __ballot(ar >= 0);
      while (active) {
        const int leader = __ffsll((long long)active) - 1;
        const int key = __shfl(ar, leader);
        const unsigned long long peers = __ballot(ar == key) & active;
        if (lane == leader) atomicAdd(&tok_cnt[key], __popcll(peers));
        active &= ~peers;
      }
    }
#pragma unroll
    for (int u = 0; u < kRowBatch; ++u) {
      if (u >= nr) break;
      if (p0 + u * kAlignThreads >= R) continue;
      const int e = re[u], a = ra[u];
      const int ar = (a >= 0 && a < NA) ? a : NA;
      if (e < 0 || e >= E) err |= MOELORA_DEVERR_EXPERT_ID;
      else atomicAdd(&sm.hist[e * NR + ar], 1);
    }
  }
  if (err) atomicOr(&err_all, err);
  __syncthreads();

  const AlignPlan P = align_plan_wave_ok(s) ? align_plan_wave(s, sm) : align_plan(s, sm);
  if (wv == 0) {  // start of each adapter rank's tokens: wave scans, 64 ranks at a time
    int run = 0;
    for (int a0 = 0; a0 < NR; a0 += kWave) {
      const int a = a0 + lane;
      int tot;
      const int x = wave_excl_scan(a < NR ? tok_cnt[a] : 0, &tot);
      if (a < NR) tok_base[a] = run + x;
      run += tot;
    }
  }
  __syncthreads();

  // tokens ordered by (adapter rank, token): stable ranks, 1024 at a time
  for (int c0 = 0; c0 < T; c0 += kAlignThreads) {
    const int t = c0 + tid;
    const bool valid = t < T;
    int dummy = 0;
    const int ar = valid ? adapter_rank(aid, t, NA, dummy) : -1;
    unsigned long long active = __ballot(valid);
    int rank = 0;
    while (active) {
      const int leader = __ffsll((long long)active) - 1;
      const int key = __shfl(ar, leader);
      const unsigned long long peers = __ballot(ar == key) & active;
      if (valid && ar == key) rank = __popcll(peers & lanemask_lt(lane));
      if (lane == leader) wtab[wv][key] = __popcll(peers);
      active &= ~peers;
    }
    __syncthreads();
    if (valid) {
      int pre = 0;
      for (int w2 = 0; w2 < wv; ++w2) pre += wtab[w2][ar];
      al.tok_perm[tok_base[ar] + cursor[ar] + pre + rank] = t;
    }
    __syncthreads();
    for (int b = tid; b < NR; b += kAlignThreads) {
      int sum = 0;
      for (int w2 = 0; w2 < kAlignWaves; ++w2) {
        sum += wtab[w2][b];
        wtab[w2][b] = 0;
      }
      cursor[b] += sum;
    }
    __syncthreads();
  }

  align_store(s, sm, P, al);
  for (int a = tid; a <= NR; a += kAlignThreads) al.tok_off[a] = a < NR ? tok_base[a] : T;
  if (tid == 0) *al.error = err_all;
}

// Alignment scatter: one workgroup per (expert, adapter rank) bucket writes
// the bucket's rows, in ascending row order, from its start position.  The
// rows of adapter rank a are visited token by token in tok_perm order
// (ascending token), j ascending, so the order is ascending p.
// With SHRINK, a bucket with an adapter is one LoRA segment, and after
// placing each chunk of its rows the workgroup computes their gate_up
// shrink (z = x A_gu[a][e]^T, seg_shrink) -- the shrink rides along with
// the alignment instead of running as a launch of its own, and reads the
// segment's A once.
template <bool SHRINK>
__global__ __launch_bounds__(kScatterThreads) void k_align_scatter(Shape s,
                                                                   const int *__restrict__ ids,
                                                                   AlignBufs al, SegShrinkArgs ss) {
  __shared__ int wsum[kScatterThreads / kWave];
  __shared__ int crow[SHRINK ? kScatterThreads : 1];                  // x row of each chunk row
  __shared__ float part[SHRINK ? kScatterThreads / kWave * 256 : 1];  // seg_shrink partials
  const int NR = s.NA + 1;
  const int bucket = blockIdx.x;
  const int e = bucket / NR, ar = bucket % NR;
  const int cnt = al.bucket_cnt[bucket];
  if (cnt == 0) return;
  const int base = al.bucket_base[bucket];
  const int t_lo = al.tok_off[ar], t_hi = al.tok_off[ar + 1];
  const int k = s.k;
  const int nitems = (t_hi - t_lo) * k;
  const int tid = threadIdx.x, lane = tid & (kWave - 1), wv = tid / kWave;
  // The segment's A rows are known before its rows are: one dword of each
  // of their 128-byte lines is read now, with the scatter's first loads, so
  // the shrink finds them in L2 instead of waiting for HBM after the
  // scatter (the value is only held until the end, never used).
  uint32_t touch = 0;
  const uint16_t *Aseg = nullptr;
  if constexpr (SHRINK) {
    if (ar < s.NA) {
      Aseg = static_cast<const uint16_t *>(ss.A) + ((size_t)ar * s.E + e) * s.r * ss.K;
      const size_t lines = ((size_t)s.r * ss.K * 2 + 127) / 128;
      for (size_t l = tid; l < lines; l += kScatterThreads)
        touch ^= *reinterpret_cast<const uint32_t *>(reinterpret_cast<const char *>(Aseg) + 128 * l);
    }
  }
  int running = 0;
  for (int c0 = 0; c0 < nitems && running < cnt; c0 += kScatterThreads) {
    const int i = c0 + tid;
    int p = 0;
    bool pred = false;
    if (i < nitems) {
      p = al.tok_perm[t_lo + i / k] * k + i % k;
      pred = ids[p] == e;
    }
    const unsigned long long bal = __ballot(pred);
    if (lane == 0) wsum[wv] = __popcll(bal);
    __syncthreads();
    int pre = 0, tot = 0;
#pragma unroll
    for (int w2 = 0; w2 < kScatterThreads / kWave; ++w2) {
      pre += (w2 < wv) ? wsum[w2] : 0;
      tot += wsum[w2];
    }
    const int slot = pre + __popcll(bal & lanemask_lt(lane));
    if (pred) al.sorted_rows[base + running + slot] = p;
    if constexpr (SHRINK) {
      if (ar < s.NA) {  // (uniform) a LoRA segment
        if (pred) crow[slot] = p / k;
        __syncthreads();
        seg_shrink<kScatterThreads / kWave>(static_cast<const uint16_t *>(ss.x), crow, tot, Aseg,
                                            ss.K, s.r, ss.z + (size_t)(base + running) * s.r,
                                            part);
      }
    }
    running += tot;
    __syncthreads();
  }
  if constexpr (SHRINK) asm volatile("" ::"v"(touch));
}

// Gate_up shrink of routed row p = blockIdx.x - 1, riding along with the
// routing + alignment workgroup: the workgroup routes its own token (the
// same deterministic routing as workgroup 0), then computes
// z[p] = x[t] . A_gu[a_t][e_p]^T with the whole workgroup.
template <int SLOTS, typename DT>
__device__ void route_row_shrink(const Shape &s, const float *__restrict__ logits,
                                 const int *__restrict__ ids_in, const RowShrinkArgs &rs,
                                 float *red) {
  __shared__ int s_e;
  const int tid = threadIdx.x, lane = tid & (kWave - 1);
  const int p = blockIdx.x - 1, t = p / s.k, j = p % s.k;
  const int a = rs.adapter_ids[t];
  if (a < 0 || a >= s.NA) return;  // no adapter: nothing to shrink
  if (tid < kWave) {
    int e = -1;
    if (logits) {
      int id;
      float wt;
      route_token<SLOTS>(logits + (size_t)t * s.E, s.E, s.k, &id, &wt);
      e = __shfl(id, j);
    } else {
      e = ids_in[p];
    }
    if (lane == 0) s_e = e;
  }
  __syncthreads();
  const int e = s_e;
  if (e < 0 || e >= s.E) return;
  const DT *x = static_cast<const DT *>(rs.x) + (size_t)t * rs.K;
  const DT *A = static_cast<const DT *>(rs.A) + ((size_t)a * s.E + e) * s.r * rs.K;
  if (rs.vec)
    row_shrink<DT, true>(x, A, rs.K, s.r, rs.z + (size_t)p * s.r, red);
  else
    row_shrink<DT, false>(x, A, rs.K, s.r, rs.z + (size_t)p * s.r, red);
}

// Small batches (R <= kSmallRows routed rows): routing and the whole
// alignment in workgroup 0.  Rows are ranked inside their bucket by
// counting the earlier rows with the same key (R comparisons from LDS per
// row), which yields the same stable order as the two-kernel path.  With
// a row shrink (DT not void), workgroups 1..R shrink one routed row each.
template <int SLOTS, typename DT>
__global__ __launch_bounds__(kAlignThreads) void k_route_align_small(
    Shape s, const float *__restrict__ logits, const int *__restrict__ ids_in,
    int *__restrict__ ids_out, float *__restrict__ w_out, const int *__restrict__ aid,
    AlignBufs al, RowShrinkArgs rs) {
  __shared__ AlignSmem sm;
  __shared__ int key[kSmallRows];
  __shared__ float wts[kSmallRows];
  __shared__ int err_all;
  if constexpr (!std::is_void_v<DT>) {
    if (blockIdx.x > 0) {
      route_row_shrink<SLOTS, DT>(s, logits, ids_in, rs, reinterpret_cast<float *>(sm.hist));
      return;
    }
  }
  const int tid = threadIdx.x, lane = tid & (kWave - 1), wv = tid / kWave;
  const int E = s.E, NA = s.NA, NR = NA + 1, R = s.R, k = s.k, T = s.T;
  const int NB = E * NR;

  if (logits) {
    for (int t = wv; t < T; t += kAlignWaves) {
      int id;
      float wt;
      route_token<SLOTS>(logits + (size_t)t * E, E, k, &id, &wt);
      if (lane < k) {
        key[t * k + lane] = id;
        wts[t * k + lane] = wt;
      }
    }
  } else {
    for (int p = tid; p < R; p += kAlignThreads) key[p] = ids_in[p];
  }
  for (int i = tid; i < NB; i += kAlignThreads) sm.hist[i] = 0;
  if (tid == 0) err_all = 0;
  __syncthreads();

  // key = expert * (NA + 1) + adapter rank, or -1 for a dropped row
  int err = 0, my_key = -1, my_id = 0;
  if (tid < R) {
    my_id = key[tid];
    const int ar = adapter_rank(aid, tid / k, NA, err);
    if (my_id < 0 || my_id >= E) {
      err |= MOELORA_DEVERR_EXPERT_ID;
    } else {
      my_key = my_id * NR + ar;
      atomicAdd(&sm.hist[my_key], 1);
    }
  }
  if (err) atomicOr(&err_all, err);
  __syncthreads();
  if (tid < R) key[tid] = my_key;

  // ends with a barrier: key[] visible
  const AlignPlan P = align_plan_wave_ok(s) ? align_plan_wave(s, sm) : align_plan(s, sm);

  // stable rank inside the bucket: earlier rows with the same key
  if (my_key >= 0) {
    int rank = 0;
#pragma unroll 8
    for (int q = 0; q < tid; ++q) rank += key[q] == my_key;
    al.sorted_rows[sm.hist[my_key] + rank] = tid;  // hist holds bucket starts
    al.row_pos[tid] = sm.hist[my_key] + rank;
  }
  if (logits && tid < R) {
    ids_out[tid] = my_id;
    w_out[tid] = wts[tid];
  }
  align_store(s, sm, P, al);
  if (tid == 0) *al.error = err_all;
}

template <int SLOTS, typename DT>
hipError_t launch_small(const Shape &s, const float *logits, const int *ids, int *ids_ws,
                        float *w_ws, const int *adapter_ids, const AlignBufs &al,
                        const RowShrinkArgs &rs, int grid, hipStream_t st) {
  return launch_kernel(k_route_align_small<SLOTS, DT>, dim3(grid), dim3(kAlignThreads), 0, st, s,
                       logits, ids, ids_ws, w_ws, adapter_ids, al, rs);
}

template <int SLOTS>
hipError_t launch_route_align_t(const Shape &s, const float *logits, const int *ids, int *ids_ws,
                                float *w_ws, const int *adapter_ids, const AlignBufs &al,
                                const RowShrinkArgs *rs, const SegShrinkArgs *ss, bool bf16,
                                hipStream_t st) {
  if (s.R <= kSmallRows) {
    if (ss) return hipErrorInvalidValue;  // segment shrinks ride along with the scatter only
    if (!rs)
      return launch_small<SLOTS, void>(s, logits, ids, ids_ws, w_ws, adapter_ids, al,
                                       RowShrinkArgs{}, 1, st);
    if (bf16)
      return launch_small<SLOTS, uint16_t>(s, logits, ids, ids_ws, w_ws, adapter_ids, al, *rs,
                                           1 + s.R, st);
    return launch_small<SLOTS, float>(s, logits, ids, ids_ws, w_ws, adapter_ids, al, *rs,
                                      1 + s.R, st);
  }
  if (rs) return hipErrorInvalidValue;  // row shrinks ride along with small batches only
  if (logits) {
    hipError_t e = launch_kernel(k_route<SLOTS>, dim3((s.T + 3) / 4), dim3(256), 0, st, logits,
                                 s.T, s.E, s.k, ids_ws, w_ws);
    if (e != hipSuccess) return e;
    ids = ids_ws;
  }
  hipError_t e =
      launch_kernel(k_align_meta, dim3(1), dim3(kAlignThreads), 0, st, s, ids, adapter_ids, al);
  if (e != hipSuccess) return e;
  if (ss)
    return launch_kernel(k_align_scatter<true>, dim3(s.E * (s.NA + 1)), dim3(kScatterThreads), 0, st,
                         s, ids, al, *ss);
  return launch_kernel(k_align_scatter<false>, dim3(s.E * (s.NA + 1)), dim3(kScatterThreads), 0, st,
                       s, ids, al, SegShrinkArgs{});
}

}  // namespace

hipError_t launch_route_align(const Shape &s, const float *logits, const int *ids,
                              int *ids_ws, float *w_ws, const int *adapter_ids,
                              const AlignBufs &al, const RowShrinkArgs *rs,
                              const SegShrinkArgs *ss, bool bf16, hipStream_t st) {
#define MOELORA_RA(SL) \
  launch_route_align_t<SL>(s, logits, ids, ids_ws, w_ws, adapter_ids, al, rs, ss, bf16, st)
  if (s.E <= 64) return MOELORA_RA(1);
  if (s.E <= 128) return MOELORA_RA(2);
  if (s.E <= 256) return MOELORA_RA(4);
  return MOELORA_RA(16);
#undef MOELORA_RA
}

}  // namespace moelora
