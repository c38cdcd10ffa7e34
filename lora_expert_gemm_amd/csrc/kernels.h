// Kernel arguments and host-side launchers of the MoE-LoRA layer kernels.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

#include "../../include/moelora.h"

namespace moelora {

// Kernel resolution.  The HIP runtime loads a source file's code object and
// looks a kernel's symbol up on the first launch of that kernel on a device.
// The first forward of a plan on a device therefore runs its dispatch once
// for every kernel selection any token count of the plan can make, on this
// thread only, with tl_resolve_only set: launch_kernel then looks the
// kernel up (hipFuncGetAttributes) instead of launching it, and later
// forwards load no code at any token count.
extern thread_local bool tl_resolve_only;
template <typename F, typename... Args>
inline hipError_t launch_kernel(F kern, dim3 grid, dim3 block, size_t lds, hipStream_t st,
                                Args... args) {
  if (tl_resolve_only) {
    hipFuncAttributes fa;
    return hipFuncGetAttributes(&fa, reinterpret_cast<const void *>(kern));
  }
  hipLaunchKernelGGL(kern, grid, block, lds, st, args...);
  return hipGetLastError();
}

// Shape of one forward call (token-count dependent parts included).
struct Shape {
  int T, H, I, E, k, NA, r;
  int R;      // T * k routed rows
  int BM;     // rows per block: 16, 32, 64 or 128 (a power of two)
  int cap;    // upper bound of the padded row count
  int nblk;   // cap / BM
  int max_seg, max_tiles;
};

// Alignment arrays in the workspace.
struct AlignBufs {
  int *sorted_rows;       // [cap]
  int *block_expert;      // [nblk]
  int *seg_start;         // [E + 1]
  int *lora_seg;          // [max_seg][4]
  int *tiles;             // [max_tiles][4]
  int *block_tile_start;  // [nblk + 1]
  int *counts;            // [4]: num_padded, n_lora_seg, n_tiles, 0
  int *error;             // [1]
  int *bucket_cnt;        // [E][NA + 1] rows per (expert, adapter rank)
  int *bucket_base;       // [E][NA + 1] first sorted position of the bucket
  int *tok_perm;          // [T] tokens ordered by (adapter rank, token)
  int *tok_off;           // [NA + 2] start of each adapter rank in tok_perm
  int *row_pos;           // [R] sorted position of each routed row (small batches)
};

// Row-wise LoRA shrink riding along with another launch (small batches):
// z[p][c] = X[row p] . A[a_p][e_p][c] for every routed row p with an adapter.
struct RowShrinkArgs {
  const void *x;           // gate_up: x [T][H] by token; down: h [cap][I] by position
  const void *A;           // [NA][E][r][K]
  float *z;                // [R][r]
  const int *adapter_ids;  // [T]
  int K;                   // contraction length (H or I)
  bool vec;                // 16-byte vector loads allowed
};

// Gate_up shrink of the LoRA segments riding along with the alignment's
// scatter (larger batches): z[pos][c] = x[row at pos] . A[a][e][c].
struct SegShrinkArgs {
  const void *x;           // [T][H] bf16
  const void *A;           // [NA][E][r][K] bf16
  float *z;                // [cap][r] (one split)
  int K;                   // contraction length (H)
};

// Operands of the expert GEMM kernels.  Pointers are typed void and cast to
// the element type inside the templates.
struct GemmArgs {
  Shape s;
  const int *topk_ids;     // [R]
  const void *x;           // [T][H]
  const void *W;           // base weights of this projection (E4M3 codes for w8 variants)
  const float *wscale;     // w8: one float32 scale per weight row, [E][rows]
  const void *A;           // LoRA A of this projection (shrink kernels)
  const void *B;           // LoRA B of this projection (expand epilogue)
  const float *z;          // [split][cap][r] shrink partial sums read by the expand,
                           // or [R][r] per routed row (row mode)
  float *z_out;            // [split][cap][r] shrink partial sums written
  int split;               // workgroups sharing one shrink tile's contraction
  int shrink_waves;        // waves per shrink workgroup (4, 8 or kShrinkWaves)
  RowShrinkArgs rs;        // row mode: the down shrink riding along with down
  int row_wgs;             // row mode: leading workgroups that run rs
  int waves;               // waves per workgroup of the GEMM kernels (16 columns each)
  int down_rows;           // streaming down GEMM: weight rows per wave (16, or 32 = two tiles)
  int slots;               // streaming GEMMs: LDS ring slots per wave for the weight stream
                           // (bf16, contraction a multiple of 64); 0: loads into registers
  int ksplit;              // streaming down GEMM with the LDS ring: contraction splits, each
                           // writing its own partial y (1: none)
  int tok_share;           // LDS ring, 4-wave workgroups: the block's tokens fetched
                           // once per workgroup into a shared LDS ring (0: per wave)
  int group;               // LDS-tiled GEMMs: item order, < 0 expert-major, else column tiles
                           // per group (<= 1: none)
  int rotate;              // LDS ring: workgroups start their contraction walk at staggered
                           // slabs (weight rows a multiple of 4 KB), 0: all at slab 0
  int z2;                  // z / z_out hold bf16 rows [cap][2r] = (hi | lo) of the fp32 shrink
                           // result (tiled shrink -> 8-wave GEMM); zero_row: 64 bf16 zeros
  void *zero_row;
  void *h;                 // [cap][I] SiLU(gate)*up, layer dtype
  float *y;                // [ksplit][R][H] down output per routed row (partials)
  AlignBufs al;
};

// Workgroup -> (block, column tile).  The grid is sized for every block
// the token count could need, but only the first num_padded / BM blocks
// hold rows (the rest would exit at once).  Workgroups are dealt round the
// 8 XCDs (workgroup b on XCD b % 8), so each XCD takes an equal, contiguous
// share of the live (block, column tile) items, in an order where the
// blocks of one column tile are consecutive (the blocks of one expert share
// an XCD and its L2); workgroups past their XCD's share get blk = -1.  (A
// contiguous split of the whole grid, empty blocks included, gave some
// XCDs a third more live work than others: the 128-expert gate_up kept all
// slots busy for only ~60 % of the launch.)  The grid is a multiple of 8.
struct GemmTile {
  int blk, nt;
};
__device__ __forceinline__ GemmTile gemm_tile(const GemmArgs &a, int bid, int ncols) {
  constexpr int kXcd = 8;
  const int nreal = a.al.counts[0] / a.s.BM;
  const int n = nreal * ncols;
  const int per = (n + kXcd - 1) / kXcd;
  const int x = bid % kXcd, j = bid / kXcd, L = x * per + j;
  if (j >= per || L >= n) return {-1, 0};
  return {L % nreal, L / nreal};
}
// The LDS-tiled GEMMs (one workgroup per CU, 32 per XCD at a time) order
// the items in groups of G column tiles instead (GemmArgs::group = G > 1):
// group g holds column tiles gG .. gG+G-1 (the last group what is left),
// its items ordered by block, then column tile.  The workgroups an XCD runs
// at once then cover about 32 / G blocks x G column tiles: each weight tile
// is shared through L2 by the blocks of its expert, and each block's token
// rows by G column tiles (block-major order shares the weights only, column
// tile-major order the tokens only).
__device__ __forceinline__ GemmTile gemm_tile_grouped(const GemmArgs &a, int bid, int ncols, int G) {
  constexpr int kXcd = 8;
  const int nreal = a.al.counts[0] / a.s.BM;
  const int n = nreal * ncols;
  const int per = (n + kXcd - 1) / kXcd;
  const int x = bid % kXcd, j = bid / kXcd, L = x * per + j;
  if (j >= per || L >= n) return {-1, 0};
  const int full = ncols / G, Lf = full * G * nreal;
  if (L < Lf) {
    const int g = L / (G * nreal), r = L - g * G * nreal;
    return {r / G, g * G + r % G};
  }
  const int Gw = ncols - full * G, r = L - Lf;
  return {r / Gw, full * G + r % Gw};
}
// Expert-major order (GemmArgs::group < 0): an expert's items sit
// together, column tile outer and block inner, so the blocks that share a
// weight tile are consecutive items (the XCD runs them at about the same
// time); an expert's first block is seg_start[e] / BM.
__device__ __forceinline__ GemmTile gemm_tile_expert(const GemmArgs &a, int bid, int ncols) {
  constexpr int kXcd = 8;
  const int BM = a.s.BM;
  const int nreal = a.al.counts[0] / BM;
  const int n = nreal * ncols;
  const int per = (n + kXcd - 1) / kXcd;
  const int x = bid % kXcd, j = bid / kXcd, L = x * per + j;
  if (j >= per || L >= n) return {-1, 0};
  const int e = a.al.block_expert[L / ncols];  // a block of the item's expert
  const int fb = a.al.seg_start[e] / BM, nb = a.al.seg_start[e + 1] / BM - fb;
  const int r = L - fb * ncols;
  return {fb + r % nb, r / nb};
}
__host__ __device__ constexpr int round_up8(int v) { return (v + 7) / 8 * 8; }
// Row pitch in bytes of E4M3 base weights with contraction length K: rows
// start on 128-byte lines, so each 128-wide slab of a row is one whole line.
__host__ __device__ constexpr size_t row_pitch8(int K) { return (size_t)(K + 127) / 128 * 128; }

// LDS ring slots per wave of the streaming GEMMs' weight stream (bf16 with a
// contraction that is a multiple of 64); the launchers hold instances for
// the counts ring_slots_supported accepts, 0 meaning loads into registers.
// Two slots leave no slab of slack between a slab's wait and its reads (the
// exactness test of the wait arithmetic); three are the measured default.
constexpr int kRingSlots = 3;
inline bool ring_slots_supported(int s) { return s == 0 || s == 2 || s == 3 || s == 4; }

// Workgroups of kShareWaves waves with an LDS ring fetch the block's tokens
// once into a shared LDS ring (GemmArgs::tok_share).  Their dynamic LDS:
// the token ring (S slots of TG groups x 16 rows x 64 bf16, or x 128 bf16
// for the E4M3 stream's wider slabs), then the waves' weight rings (S slots
// of NW 16-row tiles of 2 KB each).  The block's token-row table (BM ints)
// sits in the token ring's last slot: it is only read while the waves set
// up their token addresses, before that slot is first filled (the first
// step's wait and barrier order the two), and keeping it out of the
// footprint lets a 4-slot workgroup of 16-row blocks (and a 3-slot one of
// 32-row E4M3 blocks) fit twice into a CU's 160 KB.
constexpr int kShareWaves = 4;
constexpr int shared_lds_bytes(int TG, int NW, int S, bool w8 = false) {
  return S * TG * (w8 ? 4096 : 2048) + kShareWaves * S * NW * 2048;
}
// Byte offset of the token-row table (in the token ring's last slot).
constexpr int tok_row_offset(int TG, int S, bool w8 = false) {
  return (S - 1) * TG * (w8 ? 4096 : 2048);
}

// Shrink kernels: one workgroup per LoRA tile, of kShrinkWaves waves (or 4
// or 8 when there are many tiles).
constexpr int kShrinkWaves = 16;

// Launchers (return hipGetLastError()).
// Routing (when logits is non-null; results to ids_ws / w_ws) and the
// alignment of the routed rows (caller ids when logits is null).  With rs
// non-null (small batches only) the same launch also runs the gate_up
// shrink of every routed row; with ss non-null (more than kSmallRows rows;
// bf16, 16-byte aligned rows, H a multiple of 32) the scatter computes the
// gate_up shrink of every LoRA segment.
hipError_t launch_route_align(const Shape &s, const float *logits, const int *ids,
                              int *ids_ws, float *w_ws, const int *adapter_ids,
                              const AlignBufs &al, const RowShrinkArgs *rs,
                              const SegShrinkArgs *ss, bool bf16, hipStream_t st);
// Largest routed-row count of the one-workgroup routing + alignment.
constexpr int kSmallRows = 256;

struct GemmVariant {
  bool bf16;     // element type
  int tg;        // 16-row token groups per block (BM = 16 * tg)
  bool vec;      // 16-byte vector loads allowed
  bool even_k;   // contraction length a multiple of the K step
  bool lora;     // expand epilogue on
  bool rowz;     // row mode: z indexed by routed row (gate_up) / down shrink
                 // riding along and expand moved to the combine (down)
  bool w8;       // base weights as E4M3 codes with row scales (bf16 layer,
                 // weight stream through the LDS ring only)
};
hipError_t launch_gate_up(const GemmArgs &a, const GemmVariant &v, hipStream_t st);
// LDS-tiled MFMA GEMM for 128-row blocks (bf16, 16-byte aligned rows): the
// 8-wave kernel when the contraction is a multiple of 64 and the LoRA expand
// (if any) reads z2 rows, else the 4-wave kernel.
hipError_t launch_tiled(const GemmArgs &a, bool gate_up, const GemmVariant &v, hipStream_t st);
// LDS-tiled LoRA shrink for 128-row blocks (bf16, r <= 64, r % 8 == 0, split 1);
// writes fp32 z, or z2 rows when a.z2.
hipError_t launch_tiled_shrink(const GemmArgs &a, bool from_h, hipStream_t st);
hipError_t launch_down(const GemmArgs &a, const GemmVariant &v, hipStream_t st);
// Shrink of every LoRA tile (partial sums of a.split contraction splits).
hipError_t launch_shrink(const GemmArgs &a, const GemmVariant &v, bool from_h, hipStream_t st);
// out[t] = sum_j w[t][j] * (y[p] + [row mode] z_d[p] . B_d[a][e]^T), p = t*k + j,
// where y[p] is the sum of the ksplit partials y[0][p] + y[1][p] + ... in order.
hipError_t launch_combine(const Shape &s, const int *ids, const float *w, const float *y, int ksplit,
                          void *out, bool bf16, const float *z_d, const void *B_d,
                          const int *adapter_ids, bool vec, hipStream_t st);

}  // namespace moelora
