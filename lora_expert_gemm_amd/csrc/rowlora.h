// Row-wise LoRA pieces for decode-sized batches (a few routed rows per
// expert).  There a shrink has one row per (adapter, expert) pair, so it is
// a set of independent skinny GEMVs z[p] = x A[a][e]^T that can run in the
// same launch as other work instead of in a serial kernel of its own.
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

}  // namespace moelora
