// Grouped expert GEMMs with fused multi-LoRA for gfx950.
//
// The four LoRA ops of every expert (gate_up shrink / expand, down shrink /
// expand) and the two base projections follow the AWS ML blog "Efficiently
// serve dozens of fine-tuned models with vLLM on Amazon SageMaker AI and
// Amazon Bedrock": section "Implementing multi-LoRA inference for MoE models
// in vLLM" (one GEMM per expert, y = xW + xAB, shrink z = xA then expand zB,
// four ops per expert, per adapter, per request) and section "Kernel
// optimizations" (split-K for the skinny shrink with the partial sums
// combined afterwards; an EVEN_K instance without masks when the contraction
// length is a multiple of the step; the expand added straight into the base
// output instead of a separate pass).
//
// MFMA orientation.  Weight rows sit on the 16-row side of every MFMA and
// the block's tokens on the 16-column side, so a decode block with one or
// two tokens still fills the matrix core's rows with weights (the operand
// swap of the aib.vote news item on SageMaker MoE kernel optimizations,
// first item), and each weight element is loaded once, straight into the
// register that feeds the MFMA.  The contraction index inside a chunk is
// never interpreted: A and B chunks of a lane always cover the same indices.
//
// Work decomposition.  gate_up and down: one workgroup per (16 * waves
// output columns, BM-row block); the expert's weight tile streams through
// once per block, and blocks of the same expert sit on the same XCD so a
// second block finds the tile in L2.  Small workgroups (one or two waves)
// keep thousands of them in flight, which is what the weight stream of a
// decode step needs.  Shrink: one workgroup per LoRA tile; its waves split
// the (16-row group of A, token group, contraction) work, and when the
// contraction is split the partial sums meet in LDS and are added in a
// fixed order, so results never depend on scheduling.
#include "common.h"
#include "kernels.h"

namespace moelora {

namespace {

template <typename DT, bool VEC>
__device__ __forceinline__ u32x4_t ld(const DT *row, int k, int len) {
  if (VEC) return load_chunk(row, k);
  return load_chunk_masked(row, k, len);
}

// acc[tg] += W_rows . X_rows^T over the contraction [0, K) for one or two
// weight row pointers (TWO: gate and up), U steps of loads in flight.
// Token rows with ok false contribute zeros.
template <typename DT, int TG, int U, bool VEC, bool EVEN_K, bool TWO>
__device__ __forceinline__ void contract(const DT *w0, const DT *w1, const DT *const *xr,
                                         const bool *ok, int K, int kg, f32x4_t *acc0,
                                         f32x4_t *acc1) {
  using M = Mma<DT>;
  constexpr int EPC = Elem<DT>::kPerChunk;
  constexpr int KS = M::kK;
  const int nfull = K / KS;
  int st = 0;
  for (; st + U <= nfull; st += U) {
    u32x4_t a0[U], a1[U], b[U][TG];
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int k = (st + u) * KS + kg * EPC;
      a0[u] = ld<DT, VEC>(w0, k, K);
      if (TWO) a1[u] = ld<DT, VEC>(w1, k, K);
#pragma unroll
      for (int tg = 0; tg < TG; ++tg)
        b[u][tg] = ok[tg] ? ld<DT, VEC>(xr[tg], k, K) : u32x4_t{0, 0, 0, 0};
    }
#pragma unroll
    for (int u = 0; u < U; ++u)
#pragma unroll
      for (int tg = 0; tg < TG; ++tg) {
        M::step(acc0[tg], a0[u], b[u][tg]);
        if (TWO) M::step(acc1[tg], a1[u], b[u][tg]);
      }
  }
  for (; st < nfull; ++st) {
    const int k = st * KS + kg * EPC;
    const u32x4_t a0 = ld<DT, VEC>(w0, k, K);
    const u32x4_t a1 = TWO ? ld<DT, VEC>(w1, k, K) : a0;
#pragma unroll
    for (int tg = 0; tg < TG; ++tg) {
      const u32x4_t b = ok[tg] ? ld<DT, VEC>(xr[tg], k, K) : u32x4_t{0, 0, 0, 0};
      M::step(acc0[tg], a0, b);
      if (TWO) M::step(acc1[tg], a1, b);
    }
  }
  if (!EVEN_K) {  // the masked tail step: K is not a multiple of the step
    const int k = nfull * KS + kg * EPC;
    const u32x4_t a0 = load_chunk_any<DT, VEC>(w0, k, K);
    const u32x4_t a1 = TWO ? load_chunk_any<DT, VEC>(w1, k, K) : a0;
#pragma unroll
    for (int tg = 0; tg < TG; ++tg) {
      const u32x4_t b = ok[tg] ? load_chunk_any<DT, VEC>(xr[tg], k, K) : u32x4_t{0, 0, 0, 0};
      M::step(acc0[tg], a0, b);
      if (TWO) M::step(acc1[tg], a1, b);
    }
  }
}

// The expand of one projection, added into the base accumulators:
// acc[tg] += B_rows . z^T for the block's LoRA tiles.  z (float) feeds the
// MFMA as a bf16 hi + lo pair (a split exact to about 2^-16) or as float.
template <typename DT, int TG, bool VEC, bool TWO>
__device__ __forceinline__ void expand(const GemmArgs &a, int blk, int e, const DT *Bbase,
                                       size_t b_rows, int row, size_t row_off1, int kg, int ri,
                                       f32x4_t *acc0, f32x4_t *acc1) {
  using M = Mma<DT>;
  constexpr int EPC = Elem<DT>::kPerChunk;
  constexpr int KS = M::kK;
  constexpr int BM = 16 * TG;
  const Shape &s = a.s;
  const int r = s.r;
  const int t0 = a.al.block_tile_start[blk], t1 = a.al.block_tile_start[blk + 1];
  for (int ti = t0; ti < t1; ++ti) {
    const int4 tl = reinterpret_cast<const int4 *>(a.al.tiles)[ti];
    const int ad = tl.y, lo = tl.z, n = tl.w;
    const DT *b0 = Bbase + (((size_t)ad * s.E + e) * b_rows + row) * r;
    const DT *b1 = b0 + row_off1 * r;
    for (int kc = 0; kc < r; kc += KS) {
      const int kk = kc + kg * EPC;
      const u32x4_t c0 = load_chunk_any<DT, VEC>(b0, kk, r);
      const u32x4_t c1 = TWO ? load_chunk_any<DT, VEC>(b1, kk, r) : c0;
#pragma unroll
      for (int tg = 0; tg < TG; ++tg) {
        const int local = tg * 16 + ri;
        float zv[EPC];
#pragma unroll
        for (int q = 0; q < EPC; ++q) zv[q] = 0.f;
        if (local >= lo && local < lo + n) {
          const float *zp = a.z + ((size_t)blk * BM + local) * r + kk;
          if (VEC) {  // r is a multiple of the chunk: whole chunk in or out
            if (kk < r) {
#pragma unroll
              for (int q = 0; q < EPC; q += 4) {
                const float4 v4 = *reinterpret_cast<const float4 *>(zp + q);
                zv[q] = v4.x;
                zv[q + 1] = v4.y;
                zv[q + 2] = v4.z;
                zv[q + 3] = v4.w;
              }
            }
          } else {
#pragma unroll
            for (int q = 0; q < EPC; ++q)
              if (kk + q < r) zv[q] = zp[q];
          }
        }
        u32x4_t zh, zl;
        SplitF32<DT>::run(zv, zh, zl);
        M::step(acc0[tg], c0, zh);
        if (TWO) M::step(acc1[tg], c1, zh);
        if constexpr (sizeof(DT) == 2) {
          M::step(acc0[tg], c0, zl);
          if (TWO) M::step(acc1[tg], c1, zl);
        }
      }
    }
  }
}

// Workgroup -> (block, column tile).  Consecutive logical ids walk the
// blocks of one column tile, so the blocks of one expert share an XCD.
struct GemmTile {
  int blk, nt;
};
__device__ __forceinline__ GemmTile gemm_tile(int nblk) {
  const int L = xcd_remap(blockIdx.x, gridDim.x);
  return {L % nblk, L / nblk};
}

// gate_up GEMM + expand + SiLU(gate) * up.  Block rows are the expert's
// sorted rows; a wave's 16 h-columns n need weight rows n (gate) and I + n
// (up), so SiLU * up is formed in registers.  h is written for the block's
// real rows (padding rows are skipped by every reader).
template <typename DT, int TG, int U, bool VEC, bool EVEN_K, bool LORA>
__global__ __launch_bounds__(256) void k_gate_up(GemmArgs a) {
  constexpr int BM = 16 * TG;
  const Shape &s = a.s;
  const int lane = threadIdx.x & (kWave - 1), wave = threadIdx.x / kWave;
  const int ri = lane & 15, kg = lane >> 4;
  const GemmTile gt = gemm_tile(s.nblk);
  const int blk = gt.blk;
  const int e = a.al.block_expert[blk];  // -1 past the padded rows
  const int I = s.I, H = s.H;
  const int n0 = (gt.nt * a.waves + wave) * 16;
  if (e < 0 || n0 >= I) return;
  const int nrow = min(n0 + ri, I - 1);
  const DT *wg = static_cast<const DT *>(a.W) + ((size_t)e * 2 * I + nrow) * H;
  const DT *wu = wg + (size_t)I * H;
  const DT *xr[TG];
  bool ok[TG];
#pragma unroll
  for (int tg = 0; tg < TG; ++tg) {
    const int p = a.al.sorted_rows[blk * BM + tg * 16 + ri];
    ok[tg] = p < s.R;
    xr[tg] = static_cast<const DT *>(a.x) + (size_t)(ok[tg] ? p / s.k : 0) * H;
  }
  f32x4_t ag[TG], au[TG];
#pragma unroll
  for (int tg = 0; tg < TG; ++tg) {
    ag[tg] = f32x4_t{0.f, 0.f, 0.f, 0.f};
    au[tg] = f32x4_t{0.f, 0.f, 0.f, 0.f};
  }
  contract<DT, TG, U, VEC, EVEN_K, true>(wg, wu, xr, ok, H, kg, ag, au);
  if (LORA)
    expand<DT, TG, VEC, true>(a, blk, e, static_cast<const DT *>(a.B), (size_t)2 * I, nrow,
                              (size_t)I, kg, ri, ag, au);
  DT *hout = static_cast<DT *>(a.h);
  const int nb = n0 + kg * 4;
#pragma unroll
  for (int tg = 0; tg < TG; ++tg) {
    if (!ok[tg]) continue;  // padding row: never read
    const size_t pos = (size_t)blk * BM + tg * 16 + ri;
    DT hv[4];
#pragma unroll
    for (int v = 0; v < 4; ++v) hv[v] = Elem<DT>::from_f32(silu_f32(ag[tg][v]) * au[tg][v]);
    DT *dst = hout + pos * I + nb;
    if (VEC && nb + 3 < I) {
      if constexpr (sizeof(DT) == 2)
        *reinterpret_cast<uint2 *>(dst) = __builtin_bit_cast(uint2, hv);
      else
        *reinterpret_cast<float4 *>(dst) = __builtin_bit_cast(float4, hv);
    } else {
#pragma unroll
      for (int v = 0; v < 4; ++v)
        if (nb + v < I) dst[v] = hv[v];
    }
  }
}

// down GEMM + expand, written per routed row: y[p][m] (float).
template <typename DT, int TG, int U, bool VEC, bool EVEN_K, bool LORA>
__global__ __launch_bounds__(256) void k_down(GemmArgs a) {
  constexpr int BM = 16 * TG;
  const Shape &s = a.s;
  const int lane = threadIdx.x & (kWave - 1), wave = threadIdx.x / kWave;
  const int ri = lane & 15, kg = lane >> 4;
  const GemmTile gt = gemm_tile(s.nblk);
  const int blk = gt.blk;
  const int e = a.al.block_expert[blk];
  const int I = s.I, H = s.H;
  const int m0 = (gt.nt * a.waves + wave) * 16;
  if (e < 0 || m0 >= H) return;
  const int mrow = min(m0 + ri, H - 1);
  const DT *wd = static_cast<const DT *>(a.W) + ((size_t)e * H + mrow) * I;
  const DT *xr[TG];
  bool ok[TG];
  int prow[TG];
#pragma unroll
  for (int tg = 0; tg < TG; ++tg) {
    prow[tg] = a.al.sorted_rows[blk * BM + tg * 16 + ri];
    ok[tg] = prow[tg] < s.R;  // padding rows contribute nothing
    xr[tg] = static_cast<const DT *>(a.h) + ((size_t)blk * BM + tg * 16 + ri) * I;
  }
  f32x4_t acc[TG];
#pragma unroll
  for (int tg = 0; tg < TG; ++tg) acc[tg] = f32x4_t{0.f, 0.f, 0.f, 0.f};
  contract<DT, TG, U, VEC, EVEN_K, false>(wd, wd, xr, ok, I, kg, acc, acc);
  if (LORA)
    expand<DT, TG, VEC, false>(a, blk, e, static_cast<const DT *>(a.B), (size_t)H, mrow, 0, kg,
                               ri, acc, acc);
  const int mb = m0 + kg * 4;
#pragma unroll
  for (int tg = 0; tg < TG; ++tg) {
    if (!ok[tg]) continue;
    float *dst = a.y + (size_t)prow[tg] * H + mb;
    if (VEC && mb + 3 < H) {
      *reinterpret_cast<float4 *>(dst) = make_float4(acc[tg][0], acc[tg][1], acc[tg][2], acc[tg][3]);
    } else {
#pragma unroll
      for (int v = 0; v < 4; ++v)
        if (mb + v < H) dst[v] = acc[tg][v];
    }
  }
}

// LoRA shrink z = X A^T for the rows of one LoRA tile; X is x (gate_up,
// rows by token) or h (down, rows by sorted position).  One workgroup per
// tile.  Wave tasks are (16-row group of A, token group, contraction part);
// when there are fewer (row group, token group) pairs than waves, the
// contraction is split into nks parts whose partial sums go to LDS and are
// added in part order (split-K across waves; the partials are reduced by a
// second pass inside the workgroup rather than by atomics).
template <typename DT, int TG, bool VEC, bool EVEN_K, bool FROM_H>
__global__ __launch_bounds__(kShrinkWaves * kWave) void k_shrink(GemmArgs a) {
  using M = Mma<DT>;
  constexpr int EPC = Elem<DT>::kPerChunk;
  constexpr int KS = M::kK;
  constexpr int BM = 16 * TG;
  // partial sums of the split contraction: [nks][16 * ntg rows][r], at most
  // kShrinkWaves * 16 * 16 floats (r <= 16 * ncg and nks * ncg * ntg <= waves)
  __shared__ float part[kShrinkWaves * 16 * 16];
  const Shape &s = a.s;
  const int tile = blockIdx.x;
  if (tile >= a.al.counts[2]) return;
  const int4 tl = reinterpret_cast<const int4 *>(a.al.tiles)[tile];
  const int blk = tl.x, ad = tl.y, lo = tl.z, n = tl.w;
  const int e = a.al.block_expert[blk];
  const int lane = threadIdx.x & (kWave - 1), wave = threadIdx.x / kWave;
  const int ri = lane & 15, kg = lane >> 4;
  const int r = s.r;
  const int K = FROM_H ? s.I : s.H;
  const int ncg = (r + 15) / 16;
  const int tg_lo = lo / 16, tg_hi = (lo + n - 1) / 16, ntg = tg_hi - tg_lo + 1;
  const int pairs = ncg * ntg;
  const int nks = pairs >= kShrinkWaves ? 1 : kShrinkWaves / pairs;
  const int nsteps = (K + KS - 1) / KS;

  for (int u = wave; u < pairs * nks; u += kShrinkWaves) {
    const int cg = u % ncg, tg = tg_lo + (u / ncg) % ntg, ks = u / pairs;
    const int s_beg = (int)((long long)ks * nsteps / nks);
    const int s_end = (int)((long long)(ks + 1) * nsteps / nks);
    const int crow = min(cg * 16 + ri, r - 1);
    const DT *arow = static_cast<const DT *>(a.A) + (((size_t)ad * s.E + e) * r + crow) * K;
    const int local = tg * 16 + ri;
    const bool in = local >= lo && local < lo + n;
    const size_t pos = (size_t)blk * BM + local;
    const DT *xr;
    if (FROM_H) {
      xr = static_cast<const DT *>(a.h) + pos * s.I;
    } else {
      const int p = in ? a.al.sorted_rows[pos] : 0;
      xr = static_cast<const DT *>(a.x) + (size_t)(p / s.k) * s.H;
    }
    f32x4_t acc = f32x4_t{0.f, 0.f, 0.f, 0.f};
    constexpr int SU = 8;  // steps whose loads are in flight together
    for (int st0 = s_beg; st0 < s_end; st0 += SU) {
      u32x4_t av[SU], bv[SU];
#pragma unroll
      for (int u = 0; u < SU; ++u) {
        const int st = st0 + u;
        const int k = st * KS + kg * EPC;
        const bool live = st < s_end;
        const bool tail = !EVEN_K && st == nsteps - 1;
        av[u] = u32x4_t{0, 0, 0, 0};
        bv[u] = u32x4_t{0, 0, 0, 0};
        if (live) av[u] = tail ? load_chunk_any<DT, VEC>(arow, k, K) : ld<DT, VEC>(arow, k, K);
        if (live && in) bv[u] = tail ? load_chunk_any<DT, VEC>(xr, k, K) : ld<DT, VEC>(xr, k, K);
      }
#pragma unroll
      for (int u = 0; u < SU; ++u) M::step(acc, av[u], bv[u]);
    }
    // lane holds z[row local][c = cg*16 + kg*4 + v]
#pragma unroll
    for (int v = 0; v < 4; ++v) {
      const int c = cg * 16 + kg * 4 + v;
      if (c >= r) continue;
      if (nks == 1) {
        if (in) a.z_out[pos * r + c] = acc[v];
      } else {
        part[(ks * 16 * ntg + (tg - tg_lo) * 16 + ri) * r + c] = acc[v];
      }
    }
  }
  if (nks == 1) return;
  __syncthreads();
  for (int i = threadIdx.x; i < 16 * ntg * r; i += kShrinkWaves * kWave) {
    const int row = i / r, c = i % r;
    const int local = tg_lo * 16 + row;
    if (local < lo || local >= lo + n) continue;
    float sum = 0.f;
    for (int ks = 0; ks < nks; ++ks) sum += part[(ks * 16 * ntg + row) * r + c];
    a.z_out[((size_t)blk * BM + local) * r + c] = sum;
  }
}

// out[t] = sum_j w[t][j] * y[t*k + j] in ascending j (float), rounded to
// the layer dtype; rows with an out-of-range expert id add nothing.
template <typename DT>
__global__ __launch_bounds__(256) void k_combine(Shape s, const int *__restrict__ ids,
                                                 const float *__restrict__ w,
                                                 const float *__restrict__ y, DT *out) {
  const int t = blockIdx.x;
  const int m = (blockIdx.y * 256 + threadIdx.x) * 4;
  const int H = s.H;
  if (m >= H) return;
  float acc[4] = {0.f, 0.f, 0.f, 0.f};
  const bool vec = (H % 4) == 0;
  for (int j = 0; j < s.k; ++j) {
    const int p = t * s.k + j;
    const int e = ids[p];
    if (e < 0 || e >= s.E) continue;
    const float wj = w[p];
    const float *yr = y + (size_t)p * H + m;
    if (vec) {
      const float4 v = *reinterpret_cast<const float4 *>(yr);
      acc[0] += wj * v.x;
      acc[1] += wj * v.y;
      acc[2] += wj * v.z;
      acc[3] += wj * v.w;
    } else {
      for (int q = 0; q < 4; ++q)
        if (m + q < H) acc[q] += wj * yr[q];
    }
  }
  DT *o = out + (size_t)t * H + m;
  for (int q = 0; q < 4; ++q)
    if (m + q < H) o[q] = Elem<DT>::from_f32(acc[q]);
}

// ------------------------------------------------------------- dispatch

// K-loop unroll: deep for 16-row blocks (weight streaming), shallower for
// 64-row blocks (more accumulators).
template <int TG> constexpr int unroll_for() { return TG == 1 ? 8 : 4; }

template <typename DT, int TG, bool VEC, bool EK, bool LORA>
hipError_t go_gate_up(const GemmArgs &a, hipStream_t st) {
  const int cols = 16 * a.waves;
  const int ntn = (a.s.I + cols - 1) / cols;
  hipLaunchKernelGGL((k_gate_up<DT, TG, unroll_for<TG>(), VEC, EK, LORA>),
                     dim3(ntn * a.s.nblk), dim3(kWave * a.waves), 0, st, a);
  return hipGetLastError();
}
template <typename DT, int TG, bool VEC, bool EK, bool LORA>
hipError_t go_down(const GemmArgs &a, hipStream_t st) {
  const int cols = 16 * a.waves;
  const int ntn = (a.s.H + cols - 1) / cols;
  hipLaunchKernelGGL((k_down<DT, TG, unroll_for<TG>(), VEC, EK, LORA>),
                     dim3(ntn * a.s.nblk), dim3(kWave * a.waves), 0, st, a);
  return hipGetLastError();
}
template <typename DT, int TG, bool VEC, bool EK, bool FROM_H>
hipError_t go_shrink(const GemmArgs &a, hipStream_t st) {
  hipLaunchKernelGGL((k_shrink<DT, TG, VEC, EK, FROM_H>), dim3(a.s.max_tiles),
                     dim3(kShrinkWaves * kWave), 0, st, a);
  return hipGetLastError();
}

// (vec, even_k) in {(1,1), (1,0), (0,0)}: unaligned rows always mask.
#define MOELORA_PICK(GO, DT, TG, V, L)                                               \
  ((V).vec ? ((V).even_k ? ((L) ? GO<DT, TG, true, true, true>(a, st)                \
                                : GO<DT, TG, true, true, false>(a, st))              \
                         : ((L) ? GO<DT, TG, true, false, true>(a, st)               \
                                : GO<DT, TG, true, false, false>(a, st)))            \
           : ((L) ? GO<DT, TG, false, false, true>(a, st)                            \
                  : GO<DT, TG, false, false, false>(a, st)))

#define MOELORA_BY_TG(GO, V, L)                                                      \
  switch ((V).tg) {                                                                 \
    case 1:                                                                         \
      return (V).bf16 ? MOELORA_PICK(GO, uint16_t, 1, V, L) : MOELORA_PICK(GO, float, 1, V, L); \
    case 4:                                                                         \
      return (V).bf16 ? MOELORA_PICK(GO, uint16_t, 4, V, L) : MOELORA_PICK(GO, float, 4, V, L); \
    default:                                                                        \
      return hipErrorInvalidValue;                                                  \
  }

}  // namespace

hipError_t launch_gate_up(const GemmArgs &a, const GemmVariant &v, hipStream_t st) {
  if (a.s.nblk == 0) return hipSuccess;
  if (a.waves < 1 || a.waves > 4) return hipErrorInvalidValue;
  MOELORA_BY_TG(go_gate_up, v, v.lora)
}

hipError_t launch_down(const GemmArgs &a, const GemmVariant &v, hipStream_t st) {
  if (a.s.nblk == 0) return hipSuccess;
  if (a.waves < 1 || a.waves > 4) return hipErrorInvalidValue;
  MOELORA_BY_TG(go_down, v, v.lora)
}

hipError_t launch_shrink(const GemmArgs &a, const GemmVariant &v, bool from_h, hipStream_t st) {
  if (a.s.max_tiles == 0) return hipSuccess;
  MOELORA_BY_TG(go_shrink, v, from_h)
}

hipError_t launch_combine(const Shape &s, const int *ids, const float *w, const float *y,
                          void *out, bool bf16, hipStream_t st) {
  if (s.T == 0) return hipSuccess;
  dim3 grid(s.T, (s.H + 1023) / 1024);
  if (bf16)
    hipLaunchKernelGGL(k_combine<uint16_t>, grid, dim3(256), 0, st, s, ids, w, y,
                       static_cast<uint16_t *>(out));
  else
    hipLaunchKernelGGL(k_combine<float>, grid, dim3(256), 0, st, s, ids, w, y,
                       static_cast<float *>(out));
  return hipGetLastError();
}

}  // namespace moelora
