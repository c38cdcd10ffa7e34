// Grouped expert GEMMs with fused multi-LoRA for gfx950.
//
// The four LoRA ops of every expert (gate_up shrink / expand, down shrink /
// expand) and the two base projections follow the AWS ML blog "Efficiently
// serve dozens of fine-tuned models with vLLM on Amazon SageMaker AI and
// Amazon Bedrock": section "Implementing multi-LoRA inference for MoE models
// in vLLM" (one GEMM per expert, y = xW + xAB, shrink z = xA then expand zB,
// four ops per expert, per adapter, per request) and section "Kernel
// optimizations" (split-K for the skinny shrink, partial sums combined
// afterwards; an EVEN_K instance without masks when the contraction length
// is a multiple of the block; the expand added straight into the base
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
// Work decomposition.  gate_up and down: one workgroup per (64 output
// columns, BM-row block); the expert's weight tile streams through once per
// block, and blocks of the same expert sit on the same XCD so a second
// block finds the tile in L2.  Shrink: one workgroup per (LoRA tile, K
// split), four waves over (16-row group of A, K sub-range); every partial
// sum is written to its own slot and the expand epilogue adds the slots in
// a fixed order, so results do not depend on scheduling.
#include "common.h"
#include "kernels.h"

namespace moelora {

namespace {

constexpr int kThreads = 256;
constexpr int kUnroll = 4;

template <typename DT, bool VEC>
__device__ __forceinline__ u32x4_t ld_w(const DT *row, int k, int len) {
  if (VEC) return load_chunk_stream(row, k);
  return load_chunk_masked(row, k, len);
}

template <typename DT, bool VEC>
__device__ __forceinline__ u32x4_t ld_x(const DT *row, int k, int len) {
  if (VEC) return load_chunk(row, k);
  return load_chunk_masked(row, k, len);
}

// acc[tg] += W_rows . X_rows^T over the contraction [0, K) for one or two
// weight row pointers (TWO: gate and up).  Token rows with tok_ok false
// contribute zeros.
template <typename DT, int TG, bool VEC, bool EVEN_K, bool TWO>
__device__ __forceinline__ void contract(const DT *w0, const DT *w1, const DT *const *xr,
                                         const bool *tok_ok, int K, int kg, f32x4_t *acc0,
                                         f32x4_t *acc1) {
  using M = Mma<DT>;
  constexpr int EPC = Elem<DT>::kPerChunk;
  constexpr int KS = M::kK;
  const int nfull = K / KS;
  int st = 0;
  for (; st + kUnroll <= nfull; st += kUnroll) {
    u32x4_t a0[kUnroll], a1[kUnroll], b[kUnroll][TG];
#pragma unroll
    for (int u = 0; u < kUnroll; ++u) {
      const int k = (st + u) * KS + kg * EPC;
      a0[u] = ld_w<DT, VEC>(w0, k, K);
      if (TWO) a1[u] = ld_w<DT, VEC>(w1, k, K);
#pragma unroll
      for (int tg = 0; tg < TG; ++tg)
        b[u][tg] = tok_ok[tg] ? ld_x<DT, VEC>(xr[tg], k, K) : u32x4_t{0, 0, 0, 0};
    }
#pragma unroll
    for (int u = 0; u < kUnroll; ++u)
#pragma unroll
      for (int tg = 0; tg < TG; ++tg) {
        M::step(acc0[tg], a0[u], b[u][tg]);
        if (TWO) M::step(acc1[tg], a1[u], b[u][tg]);
      }
  }
  for (; st < nfull; ++st) {
    const int k = st * KS + kg * EPC;
    const u32x4_t a0 = ld_w<DT, VEC>(w0, k, K);
    const u32x4_t a1 = TWO ? ld_w<DT, VEC>(w1, k, K) : a0;
#pragma unroll
    for (int tg = 0; tg < TG; ++tg) {
      const u32x4_t b = tok_ok[tg] ? ld_x<DT, VEC>(xr[tg], k, K) : u32x4_t{0, 0, 0, 0};
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
      const u32x4_t b =
          tok_ok[tg] ? load_chunk_any<DT, VEC>(xr[tg], k, K) : u32x4_t{0, 0, 0, 0};
      M::step(acc0[tg], a0, b);
      if (TWO) M::step(acc1[tg], a1, b);
    }
  }
}

// The expand of one projection, added into the base accumulators:
// acc[tg] += B_rows . z^T for the block's LoRA tiles, z summed over the
// shrink partials.  z feeds the MFMA as a bf16 hi + lo pair (exact split to
// about 2^-16) or as float.
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
          const size_t pos = (size_t)blk * BM + local;
          for (int part = 0; part < a.n_part; ++part) {
            const float *zp = a.z + ((size_t)part * s.cap + pos) * r;
#pragma unroll
            for (int q = 0; q < EPC; ++q)
              if (kk + q < r) zv[q] += zp[kk + q];
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

// gate_up GEMM + expand + SiLU(gate) * up.  Block rows are the expert's
// sorted rows; the workgroup's 64 h-columns n need weight rows n (gate) and
// I + n (up), so SiLU * up is formed in registers.  h is written for every
// row of an active block (padding rows get zeros).
template <typename DT, int TG, bool VEC, bool EVEN_K, bool LORA>
__global__ __launch_bounds__(kThreads) void k_gate_up(GemmArgs a) {
  constexpr int BM = 16 * TG;
  const Shape &s = a.s;
  const int lane = threadIdx.x & (kWave - 1), wave = threadIdx.x / kWave;
  const int ri = lane & 15, kg = lane >> 4;
  const int L = xcd_remap(blockIdx.x, gridDim.x);
  const int blk = L % s.nblk, nt = L / s.nblk;
  if (blk * BM >= a.al.counts[0]) return;
  const int e = a.al.block_expert[blk];
  const int I = s.I, H = s.H;
  const int n0 = nt * kColsPerWg + wave * 16;
  if (n0 >= I) return;
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
  contract<DT, TG, VEC, EVEN_K, true>(wg, wu, xr, ok, H, kg, ag, au);
  if (LORA)
    expand<DT, TG, VEC, true>(a, blk, e, static_cast<const DT *>(a.B), (size_t)2 * I, nrow,
                              (size_t)I, kg, ri, ag, au);
  DT *hout = static_cast<DT *>(a.h);
  const int nb = n0 + kg * 4;
#pragma unroll
  for (int tg = 0; tg < TG; ++tg) {
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
template <typename DT, int TG, bool VEC, bool EVEN_K, bool LORA>
__global__ __launch_bounds__(kThreads) void k_down(GemmArgs a) {
  constexpr int BM = 16 * TG;
  const Shape &s = a.s;
  const int lane = threadIdx.x & (kWave - 1), wave = threadIdx.x / kWave;
  const int ri = lane & 15, kg = lane >> 4;
  const int L = xcd_remap(blockIdx.x, gridDim.x);
  const int blk = L % s.nblk, nt = L / s.nblk;
  if (blk * BM >= a.al.counts[0]) return;
  const int e = a.al.block_expert[blk];
  const int I = s.I, H = s.H;
  const int m0 = nt * kColsPerWg + wave * 16;
  if (m0 >= H) return;
  const int mrow = min(m0 + ri, H - 1);
  const DT *wd = static_cast<const DT *>(a.W) + ((size_t)e * H + mrow) * I;
  const DT *xr[TG];
  bool ok[TG];
#pragma unroll
  for (int tg = 0; tg < TG; ++tg) {
    ok[tg] = true;  // padding rows of h hold zeros
    xr[tg] = static_cast<const DT *>(a.h) + ((size_t)blk * BM + tg * 16 + ri) * I;
  }
  f32x4_t acc[TG];
#pragma unroll
  for (int tg = 0; tg < TG; ++tg) acc[tg] = f32x4_t{0.f, 0.f, 0.f, 0.f};
  contract<DT, TG, VEC, EVEN_K, false>(wd, wd, xr, ok, I, kg, acc, acc);
  if (LORA)
    expand<DT, TG, VEC, false>(a, blk, e, static_cast<const DT *>(a.B), (size_t)H, mrow, 0, kg,
                               ri, acc, acc);
  const int mb = m0 + kg * 4;
#pragma unroll
  for (int tg = 0; tg < TG; ++tg) {
    const int p = a.al.sorted_rows[blk * BM + tg * 16 + ri];
    if (p >= s.R) continue;
    float *dst = a.y + (size_t)p * H + mb;
    if (VEC && mb + 3 < H) {
      *reinterpret_cast<float4 *>(dst) = make_float4(acc[tg][0], acc[tg][1], acc[tg][2], acc[tg][3]);
    } else {
#pragma unroll
      for (int v = 0; v < 4; ++v)
        if (mb + v < H) dst[v] = acc[tg][v];
    }
  }
}

// LoRA shrink z = X A^T for the rows of one LoRA tile, over one split of
// the contraction; X is x (gate_up, rows by token) or h (down, rows by
// sorted position).  Writes partial sums z_out[part][pos][c].
template <typename DT, int TG, bool VEC, bool EVEN_K, bool FROM_H>
__global__ __launch_bounds__(kThreads) void k_shrink(GemmArgs a) {
  using M = Mma<DT>;
  constexpr int EPC = Elem<DT>::kPerChunk;
  constexpr int KS = M::kK;
  constexpr int BM = 16 * TG;
  const Shape &s = a.s;
  const int tile = blockIdx.x, split = blockIdx.y;
  if (tile >= a.al.counts[2]) return;
  const int4 tl = reinterpret_cast<const int4 *>(a.al.tiles)[tile];
  const int blk = tl.x, ad = tl.y, lo = tl.z, n = tl.w;
  const int e = a.al.block_expert[blk];
  const int lane = threadIdx.x & (kWave - 1), wave = threadIdx.x / kWave;
  const int ri = lane & 15, kg = lane >> 4;
  const int r = s.r;
  const int K = FROM_H ? s.I : s.H;
  const int ncg = (r + 15) / 16, nks = shrink_ksub(r);
  const int parts = a.split * nks;
  const int nsteps = (K + KS - 1) / KS;
  const int tg_lo = lo / 16, tg_hi = (lo + n - 1) / 16;

  const DT *xr[TG];
  bool in[TG];
#pragma unroll
  for (int tg = 0; tg < TG; ++tg) {
    const int local = tg * 16 + ri;
    in[tg] = local >= lo && local < lo + n;
    const size_t pos = (size_t)blk * BM + local;
    if (FROM_H) {
      xr[tg] = static_cast<const DT *>(a.h) + pos * s.I;
    } else {
      const int p = in[tg] ? a.al.sorted_rows[pos] : 0;
      xr[tg] = static_cast<const DT *>(a.x) + (size_t)(p / s.k) * s.H;
    }
  }

  for (int u = wave; u < ncg * nks; u += kThreads / kWave) {
    const int cg = u % ncg, ks = u / ncg;
    const int part = split * nks + ks;
    const int s_beg = (int)((long long)part * nsteps / parts);
    const int s_end = (int)((long long)(part + 1) * nsteps / parts);
    const int crow = min(cg * 16 + ri, r - 1);
    const DT *arow = static_cast<const DT *>(a.A) + (((size_t)ad * s.E + e) * r + crow) * K;
    f32x4_t acc[TG];
#pragma unroll
    for (int tg = 0; tg < TG; ++tg) acc[tg] = f32x4_t{0.f, 0.f, 0.f, 0.f};
    for (int st = s_beg; st < s_end; ++st) {
      const int k = st * KS + kg * EPC;
      const bool tail = !EVEN_K && st == nsteps - 1;
      const u32x4_t av = tail ? load_chunk_any<DT, VEC>(arow, k, K) : ld_x<DT, VEC>(arow, k, K);
#pragma unroll
      for (int tg = 0; tg < TG; ++tg) {
        if (tg < tg_lo || tg > tg_hi) continue;
        u32x4_t bv = u32x4_t{0, 0, 0, 0};
        if (in[tg]) bv = tail ? load_chunk_any<DT, VEC>(xr[tg], k, K) : ld_x<DT, VEC>(xr[tg], k, K);
        M::step(acc[tg], av, bv);
      }
    }
#pragma unroll
    for (int tg = 0; tg < TG; ++tg) {
      if (!in[tg]) continue;
      const size_t pos = (size_t)blk * BM + tg * 16 + ri;
      float *dst = a.z_out + ((size_t)part * s.cap + pos) * r;
#pragma unroll
      for (int v = 0; v < 4; ++v) {
        const int c = cg * 16 + kg * 4 + v;
        if (c < r) dst[c] = acc[tg][v];
      }
    }
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

template <typename DT, int TG, bool VEC, bool EK, bool LORA>
hipError_t go_gate_up(const GemmArgs &a, hipStream_t st) {
  const int ntn = (a.s.I + kColsPerWg - 1) / kColsPerWg;
  hipLaunchKernelGGL((k_gate_up<DT, TG, VEC, EK, LORA>), dim3(ntn * a.s.nblk), dim3(kThreads), 0,
                     st, a);
  return hipGetLastError();
}
template <typename DT, int TG, bool VEC, bool EK, bool LORA>
hipError_t go_down(const GemmArgs &a, hipStream_t st) {
  const int ntn = (a.s.H + kColsPerWg - 1) / kColsPerWg;
  hipLaunchKernelGGL((k_down<DT, TG, VEC, EK, LORA>), dim3(ntn * a.s.nblk), dim3(kThreads), 0, st,
                     a);
  return hipGetLastError();
}
template <typename DT, int TG, bool VEC, bool EK, bool FROM_H>
hipError_t go_shrink(const GemmArgs &a, hipStream_t st) {
  hipLaunchKernelGGL((k_shrink<DT, TG, VEC, EK, FROM_H>), dim3(a.s.max_tiles, a.split),
                     dim3(kThreads), 0, st, a);
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
  MOELORA_BY_TG(go_gate_up, v, v.lora)
}

hipError_t launch_down(const GemmArgs &a, const GemmVariant &v, hipStream_t st) {
  if (a.s.nblk == 0) return hipSuccess;
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
