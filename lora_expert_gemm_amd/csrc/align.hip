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

namespace moelora {

namespace {

constexpr int kAlignThreads = 1024;
constexpr int kAlignWaves = kAlignThreads / kWave;
constexpr int kMaxBuckets = 8448;   // E * (NA + 1)
constexpr int kMaxAdapterRanks = 256;  // NA + 1
constexpr int kScatterThreads = 512;
constexpr int kSmallRows = kAlignThreads / 4;  // fused route + align up to this many rows

__device__ __forceinline__ unsigned long long lanemask_lt(int lane) {
  return (1ull << lane) - 1ull;
}

// Exclusive prefix sum over the 1024 threads of the block; *total gets the
// sum.  tmp holds kAlignWaves ints.  Contains two barriers.
__device__ int block_excl_scan(int v, int *tmp, int *total) {
  const int lane = threadIdx.x & (kWave - 1), w = threadIdx.x / kWave;
  int x = v;
#pragma unroll
  for (int d = 1; d < kWave; d <<= 1) {
    int y = __shfl_up(x, d);
    if (lane >= d) x += y;
  }
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

// Router for one token, computed by one wave: the k largest logits (ties to
// the lower expert index, largest first) and their softmax over the kept
// logits.  Lane l holds experts l, l + 64, ...; each of the k rounds takes
// the wave-wide best untaken (value, index) by a butterfly reduction.  Lanes
// j < k end with the j-th pick in (*id, *wt).
constexpr int kRouteMaxPerLane = 1024 / kWave;

__device__ void route_token(const float *__restrict__ row, int E, int k, int *id, float *wt) {
  const int lane = threadIdx.x & (kWave - 1);
  const int per = (E + kWave - 1) / kWave;
  float v[kRouteMaxPerLane];
#pragma unroll
  for (int i = 0; i < kRouteMaxPerLane; ++i) {
    const int e = lane + i * kWave;
    v[i] = (i < per && e < E) ? row[e] : -__builtin_inff();
  }
  unsigned taken = 0;  // bit i: expert lane + 64 i already chosen
  float my_val = 0.f, top = 0.f;
  int my_id = 0;
  for (int j = 0; j < k; ++j) {
    float bv = -__builtin_inff();
    int bi = 0x7fffffff;
#pragma unroll
    for (int i = 0; i < kRouteMaxPerLane; ++i) {
      const int e = lane + i * kWave;
      if (i < per && e < E && !(taken >> i & 1u) && (v[i] > bv || bi == 0x7fffffff)) {
        bv = v[i];
        bi = e;
      }
    }
#pragma unroll
    for (int d = kWave / 2; d >= 1; d >>= 1) {
      const float ov = __shfl_xor(bv, d);
      const int oi = __shfl_xor(bi, d);
      if (oi != 0x7fffffff && (bi == 0x7fffffff || ov > bv || (ov == bv && oi < bi))) {
        bv = ov;
        bi = oi;
      }
    }
    if ((bi & (kWave - 1)) == lane) taken |= 1u << (bi / kWave);
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

// One wave per token.
__global__ __launch_bounds__(256) void k_route(const float *__restrict__ logits, int T, int E,
                                               int k, int *__restrict__ ids,
                                               float *__restrict__ w) {
  const int lane = threadIdx.x & (kWave - 1);
  const int t = blockIdx.x * (blockDim.x / kWave) + threadIdx.x / kWave;
  if (t >= T) return;
  int id;
  float wt;
  route_token(logits + (size_t)t * E, E, k, &id, &wt);
  if (lane < k) {
    ids[(size_t)t * k + lane] = id;
    w[(size_t)t * k + lane] = wt;
  }
}

__device__ __forceinline__ int adapter_rank(const int *aid, int t, int NA, int &err) {
  if (!aid) return NA;
  const int a = aid[t];
  if (a < -1 || a >= NA) err |= MOELORA_DEVERR_ADAPTER_ID;
  return (a >= 0 && a < NA) ? a : NA;
}

struct AlignSmem {
  int hist[kMaxBuckets];  // rows per (expert, adapter rank) bucket
  int seg[1024 + 1];      // padded expert starts
  int scan_tmp[kAlignWaves];
};

// Everything that follows from the bucket histogram (in LDS): padded expert
// segments, bucket start positions (al.bucket_base / bucket_cnt), padding
// sentinels, block experts, LoRA segments and their block tiles, the first
// tile of every block, and the counts.  All 1024 threads call it.
__device__ void align_layout(const Shape &s, AlignSmem &sm, const AlignBufs &al) {
  const int tid = threadIdx.x;
  const int E = s.E, NA = s.NA, NR = NA + 1, BM = s.BM, R = s.R;
  int *hist = sm.hist, *seg = sm.seg;

  // padded expert segments (E <= 1024: one expert per thread)
  int padded = 0;
  if (tid < E) {
    int c = 0;
    for (int a = 0; a < NR; ++a) c += hist[tid * NR + a];
    padded = (c + BM - 1) / BM * BM;
  }
  int num_padded;
  const int excl = block_excl_scan(padded, sm.scan_tmp, &num_padded);
  if (tid < E) seg[tid] = excl;
  if (tid == 0) seg[E] = num_padded;
  __syncthreads();
  for (int i = tid; i <= E; i += kAlignThreads) al.seg_start[i] = seg[i];

  if (tid < E) {
    int run = seg[tid];
    for (int a = 0; a < NR; ++a) {
      const int b = tid * NR + a;
      al.bucket_base[b] = run;
      al.bucket_cnt[b] = hist[b];
      run += hist[b];
    }
    for (int i = run; i < seg[tid + 1]; ++i) al.sorted_rows[i] = R;
    for (int b = seg[tid] / BM; b < seg[tid + 1] / BM; ++b) al.block_expert[b] = tid;
  }
  for (int i = num_padded + tid; i < s.cap; i += kAlignThreads) al.sorted_rows[i] = R;
  for (int b = num_padded / BM + tid; b < s.nblk; b += kAlignThreads) al.block_expert[b] = -1;
  __syncthreads();  // bucket_base visible to the whole workgroup

  // LoRA segments (expert, adapter >= 0) and their block tiles: each thread
  // owns a contiguous range of the E * NA flags.
  const int nf = E * NA;
  const int per = (nf + kAlignThreads - 1) / kAlignThreads;
  const int f0 = min(nf, tid * per), f1 = min(nf, f0 + per);
  int my_seg = 0, my_tiles = 0;
  for (int f = f0; f < f1; ++f) {
    const int b = (f / NA) * NR + f % NA;
    const int c = hist[b];
    if (c > 0) {
      const int st = al.bucket_base[b];
      ++my_seg;
      my_tiles += (st + c - 1) / BM - st / BM + 1;
    }
  }
  int n_seg, n_tiles;
  int seg_i = block_excl_scan(my_seg, sm.scan_tmp, &n_seg);
  int tile_i = block_excl_scan(my_tiles, sm.scan_tmp, &n_tiles);
  for (int f = f0; f < f1; ++f) {
    const int e = f / NA, a = f % NA, b = e * NR + a;
    const int c = hist[b];
    if (c <= 0) continue;
    const int st = al.bucket_base[b], en = st + c;
    reinterpret_cast<int4 *>(al.lora_seg)[seg_i++] = make_int4(e, a, st, c);
    for (int blk = st / BM; blk <= (en - 1) / BM; ++blk) {
      const int lo = max(st, blk * BM), hi = min(en, (blk + 1) * BM);
      reinterpret_cast<int4 *>(al.tiles)[tile_i++] = make_int4(blk, a, lo - blk * BM, hi - lo);
    }
  }
  for (int i = n_seg + tid; i < s.max_seg; i += kAlignThreads)
    reinterpret_cast<int4 *>(al.lora_seg)[i] = make_int4(-1, -1, 0, 0);
  for (int i = n_tiles + tid; i < s.max_tiles; i += kAlignThreads)
    reinterpret_cast<int4 *>(al.tiles)[i] = make_int4(-1, -1, 0, 0);
  __syncthreads();  // tiles visible

  for (int i = tid; i < n_tiles; i += kAlignThreads) {
    const int bi = al.tiles[4 * i];
    const int bp = i ? al.tiles[4 * (i - 1)] : -1;
    for (int b = bp + 1; b <= bi; ++b) al.block_tile_start[b] = i;
  }
  {
    const int last = n_tiles ? al.tiles[4 * (n_tiles - 1)] : -1;
    for (int b = last + 1 + tid; b <= s.nblk; b += kAlignThreads) al.block_tile_start[b] = n_tiles;
  }
  if (tid == 0) {
    al.counts[0] = num_padded;
    al.counts[1] = n_seg;
    al.counts[2] = n_tiles;
    al.counts[3] = 0;
  }
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

  const int tid = threadIdx.x, lane = tid & (kWave - 1), wv = tid / kWave;
  const int E = s.E, NA = s.NA, NR = NA + 1, R = s.R, k = s.k, T = s.T;
  const int NB = E * NR;

  for (int i = tid; i < NB; i += kAlignThreads) sm.hist[i] = 0;
  for (int i = tid; i < NR; i += kAlignThreads) {
    tok_cnt[i] = 0;
    cursor[i] = 0;
  }
  for (int i = tid; i < kAlignWaves * NR; i += kAlignThreads) wtab[i / NR][i % NR] = 0;
  if (tid == 0) *al.error = 0;
  __syncthreads();

  int err = 0;
  for (int t = tid; t < T; t += kAlignThreads) atomicAdd(&tok_cnt[adapter_rank(aid, t, NA, err)], 1);
  for (int p = tid; p < R; p += kAlignThreads) {
    const int e = ids[p];
    if (e < 0 || e >= E) {
      err |= MOELORA_DEVERR_EXPERT_ID;
      continue;
    }
    int dummy = 0;
    atomicAdd(&sm.hist[e * NR + adapter_rank(aid, p / k, NA, dummy)], 1);
  }
  if (err) atomicOr(al.error, err);
  __syncthreads();

  align_layout(s, sm, al);

  if (tid == 0) {
    int run = 0;
    for (int a = 0; a < NR; ++a) {
      tok_base[a] = run;
      al.tok_off[a] = run;
      run += tok_cnt[a];
    }
    al.tok_off[NR] = run;
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
}

// Alignment scatter: one workgroup per (expert, adapter rank) bucket writes
// the bucket's rows, in ascending row order, from its start position.  The
// rows of adapter rank a are visited token by token in tok_perm order
// (ascending token), j ascending, so the order is ascending p.
__global__ __launch_bounds__(kScatterThreads) void k_align_scatter(Shape s,
                                                                   const int *__restrict__ ids,
                                                                   AlignBufs al) {
  __shared__ int wsum[kScatterThreads / kWave];
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
    if (pred) al.sorted_rows[base + running + pre + __popcll(bal & lanemask_lt(lane))] = p;
    running += tot;
    __syncthreads();
  }
}

// Small batches (R <= kSmallRows routed rows): routing and the whole
// alignment in one workgroup.  Rows are ranked inside their bucket by
// counting the earlier rows with the same key (R comparisons from LDS per
// row), which yields the same stable order as the two-kernel path.
__global__ __launch_bounds__(kAlignThreads) void k_route_align_small(
    Shape s, const float *__restrict__ logits, const int *__restrict__ ids_in,
    int *__restrict__ ids_out, float *__restrict__ w_out, const int *__restrict__ aid,
    AlignBufs al) {
  __shared__ AlignSmem sm;
  __shared__ int key[kSmallRows];
  const int tid = threadIdx.x, lane = tid & (kWave - 1), wv = tid / kWave;
  const int E = s.E, NA = s.NA, NR = NA + 1, R = s.R, k = s.k, T = s.T;
  const int NB = E * NR;

  if (logits) {
    for (int t = wv; t < T; t += kAlignWaves) {
      int id;
      float wt;
      route_token(logits + (size_t)t * E, E, k, &id, &wt);
      if (lane < k) {
        ids_out[t * k + lane] = id;
        w_out[t * k + lane] = wt;
        key[t * k + lane] = id;
      }
    }
  } else {
    for (int p = tid; p < R; p += kAlignThreads) key[p] = ids_in[p];
  }
  for (int i = tid; i < NB; i += kAlignThreads) sm.hist[i] = 0;
  if (tid == 0) *al.error = 0;
  __syncthreads();

  // key = expert * (NA + 1) + adapter rank, or -1 for a dropped row
  int err = 0;
  int my_key = -1;
  if (tid < R) {
    const int e = key[tid];
    const int ar = adapter_rank(aid, tid / k, NA, err);
    if (e < 0 || e >= E) {
      err |= MOELORA_DEVERR_EXPERT_ID;
    } else {
      my_key = e * NR + ar;
      atomicAdd(&sm.hist[my_key], 1);
    }
  }
  if (err) atomicOr(al.error, err);
  __syncthreads();
  if (tid < R) key[tid] = my_key;

  align_layout(s, sm, al);  // contains barriers: key[] is visible after it

  if (my_key >= 0) {
    int rank = 0;
    for (int q = 0; q < tid; ++q) rank += key[q] == my_key;
    al.sorted_rows[al.bucket_base[my_key] + rank] = tid;
  }
}

}  // namespace

hipError_t launch_route_align(const Shape &s, const float *logits, const int *ids,
                              int *ids_ws, float *w_ws, const int *adapter_ids,
                              const AlignBufs &al, hipStream_t st) {
  if (s.R <= kSmallRows) {
    hipLaunchKernelGGL(k_route_align_small, dim3(1), dim3(kAlignThreads), 0, st, s, logits, ids,
                       ids_ws, w_ws, adapter_ids, al);
    return hipGetLastError();
  }
  if (logits) {
    hipLaunchKernelGGL(k_route, dim3((s.T + 3) / 4), dim3(256), 0, st, logits, s.T, s.E, s.k,
                       ids_ws, w_ws);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    ids = ids_ws;
  }
  hipLaunchKernelGGL(k_align_meta, dim3(1), dim3(kAlignThreads), 0, st, s, ids, adapter_ids, al);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(k_align_scatter, dim3(s.E * (s.NA + 1)), dim3(kScatterThreads), 0, st, s,
                     ids, al);
  return hipGetLastError();
}

}  // namespace moelora
