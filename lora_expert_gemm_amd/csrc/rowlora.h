// LoRA shrink pieces that ride along with the routing / alignment launch
// instead of running as serial kernels of their own.  For decode-sized
// batches (a few routed rows per expert) a shrink has one row per (adapter,
// expert) pair: a set of independent skinny GEMVs z[p] = x A[a][e]^T
// (row_shrink).  For larger batches the alignment's scatter workgroup of an
// (expert, adapter) bucket has just placed the bucket's rows, which are one
// LoRA segment, and shrinks them against the segment's A (seg_shrink).
#pragma once

#include "common.h"
#include "kernels.h"

namespace moelora {

// z[c] = sum_k xrow[k] * A[c][k] for c < r, computed by the whole workgroup
// (blockDim.x threads, a power of two >= r).  Thread (c, j) with
// G = blockDim.x / rp threads per row (rp = r rounded up to a power of two)
// sums the 16-byte chunks j, j + G, ... of row c, so G threads read G
// consecutive chunks; the G partials meet in LDS (red, blockDim.x floats)
// and are added pairwise in a fixed tree order.  Every thread calls it.
template <typename DT, bool VEC>
__device__ void row_shrink(const DT *__restrict__ xrow, const DT *__restrict__ A, int K, int r,
                           float *__restrict__ zout, float *red) {
  constexpr int EPC = Elem<DT>::kPerChunk;
  constexpr int U = 8;  // chunks in flight per thread
  const int nt = blockDim.x, tid = threadIdx.x;
  int rp = 1;
  while (rp < r) rp <<= 1;
  const int G = nt / rp;
  const int c = tid / G, j = tid % G;
  float acc = 0.f;
  if (c < r) {
    const DT *arow = A + (size_t)c * K;
    const int nch = (K + EPC - 1) / EPC;
    for (int ch0 = j; ch0 < nch; ch0 += U * G) {
      u32x4_t av[U], xv[U];
#pragma unroll
      for (int u = 0; u < U; ++u) {
        const int k = (ch0 + u * G) * EPC;
        av[u] = xv[u] = u32x4_t{0, 0, 0, 0};
        if (k < K) {
          av[u] = load_chunk_any<DT, VEC>(arow, k, K);
          xv[u] = load_chunk_any<DT, VEC>(xrow, k, K);
        }
      }
#pragma unroll
      for (int u = 0; u < U; ++u) {
        const Chunk<DT> ca = chunk_elems<DT>(av[u]), cx = chunk_elems<DT>(xv[u]);
#pragma unroll
        for (int q = 0; q < EPC; ++q)
          acc = __builtin_fmaf(Elem<DT>::to_f32(ca.v[q]), Elem<DT>::to_f32(cx.v[q]), acc);
      }
    }
  }
  red[tid] = acc;
  __syncthreads();
  for (int h = G / 2; h > 0; h >>= 1) {
    if (j < h) red[tid] += red[tid + h];
    __syncthreads();
  }
  if (j == 0 && c < r) zout[c] = red[tid];
}

// z[i][c] = X[tok[i]] . A[c] for the n rows i < n of a LoRA segment
// (z = the segment's first row of the [cap][r] shrink output), on the
// matrix cores: wave tasks are (16-row group of A, 16-row group of the
// segment, contraction part), with the contraction cut into nks parts when
// there are fewer (A group, row group) pairs than the NWV waves; those
// partial sums meet in part (LDS, NWV * 256 floats) and are added in part
// order, so z does not depend on scheduling.  tok (LDS) holds the x row
// of each segment row.  bf16, 16-byte aligned rows, K a multiple of 32.
// Every thread of the workgroup calls it; it ends with a barrier.
template <int NWV>
__device__ void seg_shrink(const uint16_t *__restrict__ x, const int *tok, int n,
                           const uint16_t *__restrict__ A, int K, int r, float *__restrict__ z,
                           float *part) {
  using M = Mma<uint16_t>;
  constexpr int EPC = Elem<uint16_t>::kPerChunk;
  constexpr int KS = M::kK;
  const int lane = threadIdx.x & (kWave - 1), wave = threadIdx.x / kWave;
  const int ri = lane & 15, kg = lane >> 4;
  const int ncg = (r + 15) / 16, ntg = (n + 15) / 16;
  const int pairs = ncg * ntg;
  const int nks = pairs >= NWV ? 1 : NWV / pairs;
  const int nsteps = K / KS;
  for (int u = wave; u < pairs * nks; u += NWV) {
    const int cg = u % ncg, tg = (u / ncg) % ntg, ks = u / pairs;
    const int s_beg = ks * nsteps / nks, s_end = (ks + 1) * nsteps / nks;
    const uint16_t *arow = A + (size_t)min(cg * 16 + ri, r - 1) * K;
    const int local = tg * 16 + ri;
    const bool in = local < n;
    const uint16_t *xr = x + (size_t)tok[in ? local : 0] * K;
    f32x4_t acc = f32x4_t{0.f, 0.f, 0.f, 0.f};
    // steps whose loads are in flight together (four: the caller has
    // brought A into L2, and fewer registers keep more of its workgroups
    // resident)
    constexpr int SU = 4;
    for (int st0 = s_beg; st0 < s_end; st0 += SU) {
      u32x4_t av[SU], bv[SU];
#pragma unroll
      for (int q = 0; q < SU; ++q) {
        const int st = st0 + q;
        const int k = st * KS + kg * EPC;
        av[q] = bv[q] = u32x4_t{0, 0, 0, 0};
        if (st < s_end) {
          av[q] = load_chunk(arow, k);
          if (in) bv[q] = load_chunk(xr, k);
        }
      }
#pragma unroll
      for (int q = 0; q < SU; ++q) M::step(acc, av[q], bv[q]);
    }
    // lane holds z[local][c = cg * 16 + kg * 4 + v]
#pragma unroll
    for (int v = 0; v < 4; ++v) {
      const int c = cg * 16 + kg * 4 + v;
      if (c >= r) continue;
      if (nks == 1) {
        if (in) z[(size_t)local * r + c] = acc[v];
      } else {
        part[(ks * 16 * ntg + local) * r + c] = acc[v];
      }
    }
  }
  if (nks > 1) {  // (uniform)
    __syncthreads();
    for (int i = threadIdx.x; i < n * r; i += NWV * kWave) {
      const int row = i / r, c = i - row * r;
      float sum = 0.f;
      for (int ks = 0; ks < nks; ++ks) sum += part[(ks * 16 * ntg + row) * r + c];
      z[(size_t)row * r + c] = sum;
    }
  }
  __syncthreads();
}

}  // namespace moelora
