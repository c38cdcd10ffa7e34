// LDS-tiled grouped expert GEMMs for large batches (hundreds of rows per
// expert), where the layer is bound by the matrix cores, not by HBM.
//
// Same computation as the streaming kernels in expert_gemm.hip: the grouped
// gate_up / down GEMMs of the AWS ML blog "Efficiently serve dozens of
// fine-tuned models with vLLM on Amazon SageMaker AI and Amazon Bedrock",
// section "Implementing multi-LoRA inference for MoE models in vLLM" (one
// GEMM per expert), with the LoRA expand added into the base accumulators
// (section "Kernel optimizations").
//
// Two kernels, both with v_mfma_f32_32x32x16_bf16 (weights on the 32-row
// side, tokens on the 32-column side), SiLU(gate)*up formed in registers
// (a wave holds the gate rows and the matching up rows of its h-columns):
//
// k_tiled8 (contractions that are a multiple of 64): 128 tokens x 512
// weight rows, 8 waves, one workgroup per CU; 64-wide slabs fetched with
// global_load_lds_dwordx4 straight into two 80 KB LDS stages; the LoRA
// expand runs as extra slabs of the same loop.
//
// k_tiled (the rest): 128 tokens x 256 weight rows, 4 waves, sized for two
// workgroups per CU; 32-wide slabs staged through registers into double-buffered LDS
// (the loads of slab s+1 are issued before the MFMAs of slab s and written
// to the other buffer after them; one barrier per slab); the LoRA expand in
// the epilogue.
//
// LDS rows hold one slab of one weight or token row with XOR-swizzled
// 16-byte chunks.
#include "common.h"
#include "kernels.h"

namespace moelora {

namespace {

typedef float f32x16_t __attribute__((ext_vector_type(16)));

constexpr int kTM = 128;   // tokens per workgroup tile (= block size)
constexpr int kTW = 256;   // weight rows per workgroup tile
constexpr int kTWaves = 4;
constexpr int kTThreads = kTWaves * kWave;

__device__ __forceinline__ void mma32(f32x16_t &c, u32x4_t a, u32x4_t b) {
  c = __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8_t, a),
                                              __builtin_bit_cast(bf16x8_t, b), c, 0, 0, 0);
}

// LoRA expand (acc += B_rows . z^T for each LoRA tile of the block) and the
// epilogue of a tiled workgroup: 128 tokens of block blk against TW weight
// rows starting at output column n0 (gate_up: TW/2 gate rows then the
// matching TW/2 up rows).  The wave owns weight-tile rows wt0 .. wt0+31 and
// wt1 .. wt1+31 against the block's four 32-token tiles.
template <bool GATE_UP, bool LORA, int TW>
__device__ __forceinline__ void tile_finish(const GemmArgs &a, f32x16_t (&acc)[2][4], int blk, int e,
                                            int n0, int wt0, int wt1, int li, int lh) {
  const Shape &s = a.s;
  const int I = s.I, H = s.H;
  const int Nout = GATE_UP ? I : H;
  // ---- LoRA expand: acc += B_rows . z^T for each LoRA tile of the block
  if (LORA) {
    const int r = s.r;
    const uint16_t *Bm = static_cast<const uint16_t *>(a.B);
    const int t0 = a.al.block_tile_start[blk], t1 = a.al.block_tile_start[blk + 1];
    const size_t stride = (size_t)s.cap * r;
    for (int ti = t0; ti < t1; ++ti) {
      const int4 tl = reinterpret_cast<const int4 *>(a.al.tiles)[ti];
      const int ad = tl.y, lo = tl.z, n = tl.w;
      const uint16_t *bw[2];
#pragma unroll
      for (int i = 0; i < 2; ++i) {
        const int wr = (i == 0 ? wt0 : wt1) + li;
        int row;
        if (GATE_UP) row = (wr < TW / 2 ? 0 : I) + min(n0 + (wr & (TW / 2 - 1)), I - 1);
        else row = min(n0 + wr, H - 1);
        bw[i] = Bm + (((size_t)ad * s.E + e) * (GATE_UP ? 2 * I : H) + row) * r;
      }
      for (int kc = 0; kc < r; kc += 16) {
        const int kk = kc + lh * 8;
        const u32x4_t c0 = load_chunk_any<uint16_t, true>(bw[0], kk, r);
        const u32x4_t c1 = load_chunk_any<uint16_t, true>(bw[1], kk, r);
#pragma unroll
        for (int b = 0; b < 4; ++b) {
          const int local = b * 32 + li;
          float zv[8];
#pragma unroll
          for (int q = 0; q < 8; ++q) zv[q] = 0.f;
          if (local >= lo && local < lo + n && kk < r) {
            const float *zp = a.z + ((size_t)blk * kTM + local) * r + kk;
            for (int sp = 0; sp < a.split; ++sp) {
              const float4 v0 = *reinterpret_cast<const float4 *>(zp + sp * stride);
              const float4 v1 = *reinterpret_cast<const float4 *>(zp + sp * stride + 4);
              zv[0] += v0.x, zv[1] += v0.y, zv[2] += v0.z, zv[3] += v0.w;
              zv[4] += v1.x, zv[5] += v1.y, zv[6] += v1.z, zv[7] += v1.w;
            }
          }
          u32x4_t zh, zl;
          SplitF32<uint16_t>::run(zv, zh, zl);
          mma32(acc[0][b], c0, zh);
          mma32(acc[0][b], c0, zl);
          mma32(acc[1][b], c1, zh);
          mma32(acc[1][b], c1, zl);
        }
      }
    }
  }

  // ---- epilogue.  Lane holds, for token tile b, token column 32 b + li and
  // weight rows 8 (v / 4) + 4 lh + v % 4 of each of its two weight tiles.
#pragma unroll
  for (int b = 0; b < 4; ++b) {
    const int pos = blk * kTM + b * 32 + li;
    const int p = a.al.sorted_rows[pos];
    if (p >= s.R) continue;
#pragma unroll
    for (int g = 0; g < 4; ++g) {
      const int wr = 8 * g + 4 * lh;  // first of 4 consecutive rows in the wave's tile
      if (GATE_UP) {
        const int col = n0 + wt0 + wr;  // h column
        uint16_t hv[4];
#pragma unroll
        for (int v = 0; v < 4; ++v)
          hv[v] = f32_to_bf16(silu_f32(acc[0][b][4 * g + v]) * acc[1][b][4 * g + v]);
        uint16_t *dst = static_cast<uint16_t *>(a.h) + (size_t)pos * I + col;
        if (col + 3 < Nout) {
          *reinterpret_cast<uint2 *>(dst) = __builtin_bit_cast(uint2, hv);
        } else {
          for (int v = 0; v < 4; ++v)
            if (col + v < Nout) dst[v] = hv[v];
        }
      } else {
#pragma unroll
        for (int i = 0; i < 2; ++i) {
          const int m = n0 + (i == 0 ? wt0 : wt1) + wr;
          float *dst = a.y + (size_t)p * H + m;
          if (m + 3 < Nout) {
            *reinterpret_cast<float4 *>(dst) =
                make_float4(acc[i][b][4 * g], acc[i][b][4 * g + 1], acc[i][b][4 * g + 2],
                            acc[i][b][4 * g + 3]);
          } else {
            for (int v = 0; v < 4; ++v)
              if (m + v < Nout) dst[v] = acc[i][b][4 * g + v];
          }
        }
      }
    }
  }
}

template <int BK>
struct Lds {
  static constexpr int kCpr = BK / 8;                // 16-byte chunks per row
  static constexpr int kRpl = 8 / kCpr;              // rows per 128-byte line
  static constexpr int kABytes = kTW * BK * 2;
  static constexpr int kBBytes = kTM * BK * 2;
  static constexpr int kStage = kABytes + kBBytes;
  // The chunk index is XOR-swizzled by (row / kRpl + row / 8) % kCpr: the
  // 16 consecutive rows that 16 lanes read at one logical chunk then fall
  // on 16 distinct 16-byte bank groups of a 256-byte window (and 8 rows on
  // 8 groups of a 128-byte window), and a row's chunks stay a permutation.
  __device__ static int off(int row, int c) {
    return row * (BK * 2) + ((c ^ ((row / kRpl + row / 8) % kCpr)) << 4);
  }
};

// BK = 32 halves the LDS footprint (48 KB) so that two workgroups share a
// CU and hide each other's slab loads and barriers.
template <bool GATE_UP, int BK, bool EVEN_K, bool LORA>
__global__ __launch_bounds__(kTThreads, BK == 32 ? 2 : 1) void k_tiled(GemmArgs a) {
  using L = Lds<BK>;
  extern __shared__ __align__(16) unsigned char smem[];
  const Shape &s = a.s;
  const int tid = threadIdx.x, lane = tid & (kWave - 1), wave = tid / kWave;
  const int li = lane & 31, lh = lane >> 5;

  const int I = s.I, H = s.H;
  const int ncols_t = ((GATE_UP ? I : H) + (GATE_UP ? kTW / 2 : kTW) - 1) / (GATE_UP ? kTW / 2 : kTW);
  const GemmTile gt = a.group < 0 ? gemm_tile_expert(a, blockIdx.x, ncols_t) : a.group > 1 ? gemm_tile_grouped(a, blockIdx.x, ncols_t, a.group)
                                  : gemm_tile(a, blockIdx.x, ncols_t);
  if (gt.blk < 0) return;
  const int blk = gt.blk, nt = gt.nt;
  const int e = a.al.block_expert[blk];
  const int K = GATE_UP ? H : I;
  const int n0 = nt * (GATE_UP ? kTW / 2 : kTW);  // first output column of the tile

  // ---- per-thread global load plan: thread t loads chunk (t % kCpr) of
  // rows t / kCpr + j * (kTThreads / kCpr)
  constexpr int kRowStep = kTThreads / L::kCpr;
  constexpr int kALoads = kTW / kRowStep, kBLoads = kTM / kRowStep;
  const int lc = tid % L::kCpr, lr = tid / L::kCpr;
  const uint16_t *W = static_cast<const uint16_t *>(a.W);
  const uint16_t *arow[kALoads];
#pragma unroll
  for (int j = 0; j < kALoads; ++j) {
    const int r = lr + j * kRowStep;  // weight-tile row
    int wrow;
    if (GATE_UP) {
      const int col = min(n0 + (r & (kTW / 2 - 1)), I - 1);
      wrow = (r < kTW / 2 ? 0 : I) + col;
      arow[j] = W + ((size_t)e * 2 * I + wrow) * K;
    } else {
      wrow = min(n0 + r, H - 1);
      arow[j] = W + ((size_t)e * H + wrow) * K;
    }
  }
  const uint16_t *brow[kBLoads];
  bool bok[kBLoads];
#pragma unroll
  for (int j = 0; j < kBLoads; ++j) {
    const int r = lr + j * kRowStep;
    const int pos = blk * kTM + r;
    const int p = a.al.sorted_rows[pos];
    bok[j] = p < s.R;
    if (GATE_UP)
      brow[j] = static_cast<const uint16_t *>(a.x) + (size_t)(bok[j] ? p / s.k : 0) * H;
    else
      brow[j] = static_cast<const uint16_t *>(a.h) + (size_t)pos * I;
  }

  // register staging of one slab: loaded while the previous slab's MFMAs run
  struct Stage {
    u32x4_t a[kALoads], b[kBLoads];
  };
  Stage st;
  auto gload = [&](Stage &g, int ks) {
    const int k = ks * BK + lc * 8;
#pragma unroll
    for (int j = 0; j < kALoads; ++j)
      g.a[j] = EVEN_K ? load_chunk(arow[j], k) : load_chunk_any<uint16_t, true>(arow[j], k, K);
#pragma unroll
    for (int j = 0; j < kBLoads; ++j) {
      g.b[j] = u32x4_t{0, 0, 0, 0};
      if (bok[j]) g.b[j] = EVEN_K ? load_chunk(brow[j], k) : load_chunk_any<uint16_t, true>(brow[j], k, K);
    }
  };
  auto lstore = [&](const Stage &g, int buf) {
    unsigned char *sa = smem + buf * L::kStage, *sb = sa + L::kABytes;
#pragma unroll
    for (int j = 0; j < kALoads; ++j)
      *reinterpret_cast<u32x4_t *>(sa + L::off(lr + j * kRowStep, lc)) = g.a[j];
#pragma unroll
    for (int j = 0; j < kBLoads; ++j)
      *reinterpret_cast<u32x4_t *>(sb + L::off(lr + j * kRowStep, lc)) = g.b[j];
  };

  // wave's weight tiles (rows within the 256-row tile) and token tiles
  const int wt0 = GATE_UP ? wave * 32 : wave * 64;
  const int wt1 = GATE_UP ? kTW / 2 + wave * 32 : wave * 64 + 32;

  f32x16_t acc[2][4];
#pragma unroll
  for (int i = 0; i < 2; ++i)
#pragma unroll
    for (int b = 0; b < 4; ++b) acc[i][b] = f32x16_t{};

  // MFMAs of one slab from LDS buffer buf; fragments of k-step kk + 1 are
  // read while the MFMAs of kk run
  auto compute = [&](int buf) {
    const unsigned char *sa = smem + buf * L::kStage, *sb = sa + L::kABytes;
    u32x4_t fa[2][2], fb[2][4];
    auto fread = [&](int kk, int slot) {
      const int c = 2 * kk + lh;  // this lane's 16-byte chunk of the slab
      fa[slot][0] = *reinterpret_cast<const u32x4_t *>(sa + L::off(wt0 + li, c));
      fa[slot][1] = *reinterpret_cast<const u32x4_t *>(sa + L::off(wt1 + li, c));
#pragma unroll
      for (int b = 0; b < 4; ++b)
        fb[slot][b] = *reinterpret_cast<const u32x4_t *>(sb + L::off(b * 32 + li, c));
    };
    fread(0, 0);
#pragma unroll
    for (int kk = 0; kk < BK / 16; ++kk) {
      if (kk + 1 < BK / 16) fread(kk + 1, (kk + 1) & 1);
#pragma unroll
      for (int b = 0; b < 4; ++b) {
        mma32(acc[0][b], fa[kk & 1][0], fb[kk & 1][b]);
        mma32(acc[1][b], fa[kk & 1][1], fb[kk & 1][b]);
      }
    }
  };

  const int nks = (K + BK - 1) / BK;
  gload(st, 0);
  lstore(st, 0);
  __syncthreads();
  for (int ks = 0; ks < nks; ++ks) {
    const int buf = ks & 1;
    if (ks + 1 < nks) gload(st, ks + 1);
    compute(buf);
    if (ks + 1 < nks) lstore(st, buf ^ 1);
    __syncthreads();
  }

  tile_finish<GATE_UP, LORA, kTW>(a, acc, blk, e, n0, wt0, wt1, li, lh);
}

// 8-wave variant for contractions that are a multiple of 64: workgroup tile
// 128 tokens x 512 weight rows, one workgroup per CU, two waves per SIMD.
// Wave w owns weight rows 64w .. 64w+63 (gate_up: gate rows 32w .. +31 and
// the matching up rows 256 + 32w .. +31) against all 128 tokens.
//
// Slabs are 64 contraction indices wide, so a weight or token row
// contributes one whole 128-byte cache line per slab: each group of 8 lanes
// fetches one line with global_load_lds_dwordx4, straight into LDS without
// passing through registers, and every L2 request is a full line.  Two LDS
// stages of 80 KB: the loads of slab s+1 go to one while the MFMAs of slab s
// read the other; one barrier per slab.  A row's 16-byte chunk c sits at
// chunk c ^ ((row / 2) % 8) of its 128-byte LDS row, which keeps the
// fragment reads (32 rows at chunk c, 32 rows at chunk c ^ 1) free of bank
// conflicts.
constexpr int kT8Waves = 8;
constexpr int kT8Threads = kT8Waves * kWave;
constexpr int kT8W = 512;                                 // weight rows per tile
constexpr int kT8Row = 128;                               // LDS bytes per row (64 bf16)
constexpr int kT8Stage = (kT8W + kTM) * kT8Row;           // 80 KB
constexpr int kT8Lds = 2 * kT8Stage;

__device__ __forceinline__ int t8_off(int row, int c) { return row * kT8Row + ((c ^ ((row >> 1) & 7)) << 4); }

template <bool GATE_UP, bool LORA>
__global__ __launch_bounds__(kT8Threads, 1) void k_tiled8(GemmArgs a) {
  extern __shared__ __align__(16) unsigned char smem[];
  const Shape &s = a.s;
  const int tid = threadIdx.x, lane = tid & (kWave - 1), wave = tid / kWave;
  const int li = lane & 31, lh = lane >> 5;

  const int I = s.I, H = s.H;
  // blocks vary fastest: concurrent workgroups share a weight tile
  const int ncols_t = ((GATE_UP ? I : H) + (GATE_UP ? kT8W / 2 : kT8W) - 1) / (GATE_UP ? kT8W / 2 : kT8W);
  const GemmTile gt = a.group < 0 ? gemm_tile_expert(a, blockIdx.x, ncols_t) : a.group > 1 ? gemm_tile_grouped(a, blockIdx.x, ncols_t, a.group)
                                  : gemm_tile(a, blockIdx.x, ncols_t);
  if (gt.blk < 0) return;
  const int blk = gt.blk, nt = gt.nt;
  const int e = a.al.block_expert[blk];
  const int K = GATE_UP ? H : I;
  const int n0 = nt * (GATE_UP ? kT8W / 2 : kT8W);

  // Load plan: LDS row group j (8 rows, 1 KB) is filled by one wave
  // instruction, lane i bringing logical chunk (i % 8) ^ ((row / 2) % 8) of
  // row 8j + i / 8 -- the chunk that t8_off places at byte 16 i of the group.
  // Wave w fills weight groups 8w .. 8w+7 and token groups 64 + 2w, 65 + 2w.
  const int lrow = lane >> 3;
  const uint16_t *src[10];
  {
    const uint16_t *W = static_cast<const uint16_t *>(a.W);
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      const int r = 64 * wave + 8 * j + lrow;  // weight-tile row
      const int c = (lane & 7) ^ ((r >> 1) & 7);
      size_t row;
      if (GATE_UP) row = (size_t)e * 2 * I + (r < kT8W / 2 ? 0 : I) + min(n0 + (r & (kT8W / 2 - 1)), I - 1);
      else row = (size_t)e * H + min(n0 + r, H - 1);
      src[j] = W + row * K + 8 * c;
    }
#pragma unroll
    for (int j = 0; j < 2; ++j) {
      const int t = 16 * wave + 8 * j + lrow;  // token row of the block
      const int c = (lane & 7) ^ (((kT8W + t) >> 1) & 7);
      const int pos = blk * kTM + t;
      // padding rows read a valid row; their output columns are dropped
      const int p = a.al.sorted_rows[pos];
      const uint16_t *row;
      if (GATE_UP) row = static_cast<const uint16_t *>(a.x) + (size_t)(p < s.R ? p / s.k : 0) * H;
      else row = static_cast<const uint16_t *>(a.h) + (size_t)(p < s.R ? pos : blk * kTM) * I;
      src[8 + j] = row + 8 * c;
    }
  }
  // The same base-slab rows through buffer resources (the expert's weight
  // rows; x, or the block's h rows): a weight row past the valid columns of
  // the tile (the last column tile of I = 2880 holds 64 of 256) or a padding
  // token row gets an offset past its resource's end, so its load fetches
  // nothing and leaves stale bytes in its LDS row, whose outputs are
  // dropped.  The loads keep their count per slab.  Only where every
  // resource is under 2 GB, so that kOut lies past its end.
  constexpr uint32_t kOut = 0x80000000u;
  const size_t erows = GATE_UP ? (size_t)2 * I : (size_t)H;
  const size_t tbytes = GATE_UP ? (size_t)s.T * H * 2 : (size_t)kTM * I * 2;
  const bool bres = erows * K * 2 < kOut && tbytes < kOut;
  const __amdgpu_buffer_rsrc_t wres = __builtin_amdgcn_make_buffer_rsrc(
      const_cast<uint16_t *>(static_cast<const uint16_t *>(a.W)) + (size_t)e * erows * K, (short)0,
      bres ? (int)(erows * K * 2) : 0, kBufferWord3);
  const __amdgpu_buffer_rsrc_t tres = __builtin_amdgcn_make_buffer_rsrc(
      GATE_UP ? const_cast<void *>(a.x)
              : static_cast<void *>(static_cast<uint16_t *>(a.h) + (size_t)blk * kTM * I),
      (short)0, bres ? (int)tbytes : 0, kBufferWord3);
  uint32_t voff[10];
#pragma unroll
  for (int j = 0; j < 8; ++j) {
    const int r = 64 * wave + 8 * j + lrow;
    const int c = (lane & 7) ^ ((r >> 1) & 7);
    const int col = n0 + (GATE_UP ? (r & (kT8W / 2 - 1)) : r);
    const int row = GATE_UP ? (r < kT8W / 2 ? 0 : I) + col : col;  // within the expert
    voff[j] = col < (GATE_UP ? I : H) ? (uint32_t)(((size_t)row * K + 8 * c) * 2) : kOut;
  }
#pragma unroll
  for (int j = 0; j < 2; ++j) {
    const int t = 16 * wave + 8 * j + lrow;
    const int c = (lane & 7) ^ (((kT8W + t) >> 1) & 7);
    const int p = a.al.sorted_rows[blk * kTM + t];
    const size_t off = GATE_UP ? (size_t)(p / s.k) * H : (size_t)t * I;
    voff[8 + j] = p < s.R ? (uint32_t)((off + 8 * c) * 2) : kOut;
  }
  const int nbase = K / 64;
  // LoRA expand as extra slabs: for LoRA tile (adapter ad, block rows
  // lo .. lo+n-1) the contraction runs over the 2r entries (z hi | z lo) of
  // each token against (B row | B row) of each weight row; tokens outside
  // the tile's run read zeros.
  int t0 = 0, nlt = 0;
  if (LORA) {
    t0 = a.al.block_tile_start[blk];
    nlt = a.al.block_tile_start[blk + 1] - t0;
  }
  const int lsl = LORA ? s.r / 32 : 0;  // slabs per LoRA tile
  const int nks = nbase + nlt * lsl;

  auto dma = [&](const uint16_t *g, unsigned char *l) {
    __builtin_amdgcn_global_load_lds(g, (__attribute__((address_space(3))) void *)l, 16, 0, 0);
  };
  auto issue = [&](int ks, int buf) {
    unsigned char *st = smem + buf * kT8Stage;
    if (!LORA || ks < nbase) {
      const int k = ks * 64;
      if (bres) {
#pragma unroll
        for (int j = 0; j < 8; ++j)
          __builtin_amdgcn_raw_ptr_buffer_load_lds(
              wres, (__attribute__((address_space(3))) void *)(st + (64 * wave + 8 * j) * kT8Row), 16,
              voff[j], 2 * k, 0, 0);
#pragma unroll
        for (int j = 0; j < 2; ++j)
          __builtin_amdgcn_raw_ptr_buffer_load_lds(
              tres,
              (__attribute__((address_space(3))) void *)(st + (kT8W + 16 * wave + 8 * j) * kT8Row),
              16, voff[8 + j], 2 * k, 0, 0);
        return;
      }
#pragma unroll
      for (int j = 0; j < 8; ++j) dma(src[j] + k, st + (64 * wave + 8 * j) * kT8Row);
#pragma unroll
      for (int j = 0; j < 2; ++j) dma(src[8 + j] + k, st + (kT8W + 16 * wave + 8 * j) * kT8Row);
      return;
    }
    const int u = ks - nbase, q = u % lsl;
    const int4 tl = reinterpret_cast<const int4 *>(a.al.tiles)[t0 + u / lsl];
    const int ad = tl.y, lo = tl.z, n = tl.w, r = s.r, rc = r / 8;
    const uint16_t *Bm = static_cast<const uint16_t *>(a.B) +
                         ((size_t)ad * s.E + e) * (size_t)(GATE_UP ? 2 * I : H) * r;
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      const int rr = 64 * wave + 8 * j + lrow;
      const int kc = 8 * q + ((lane & 7) ^ ((rr >> 1) & 7));  // chunk of (hi | lo)
      int row;
      if (GATE_UP) row = (rr < kT8W / 2 ? 0 : I) + min(n0 + (rr & (kT8W / 2 - 1)), I - 1);
      else row = min(n0 + rr, H - 1);
      dma(Bm + (size_t)row * r + 8 * (kc % rc), st + (64 * wave + 8 * j) * kT8Row);
    }
#pragma unroll
    for (int j = 0; j < 2; ++j) {
      const int t = 16 * wave + 8 * j + lrow;
      const int c = (lane & 7) ^ ((t >> 1) & 7);
      const uint16_t *zs = (t >= lo && t < lo + n)
                               ? static_cast<const uint16_t *>(static_cast<const void *>(a.z)) +
                                     ((size_t)blk * kTM + t) * 2 * r + 64 * q + 8 * c
                               : static_cast<const uint16_t *>(a.zero_row) + 8 * c;
      dma(zs, st + (kT8W + 16 * wave + 8 * j) * kT8Row);
    }
  };

  const int wt0 = GATE_UP ? wave * 32 : wave * 64;
  const int wt1 = GATE_UP ? kT8W / 2 + wave * 32 : wave * 64 + 32;

  f32x16_t acc[2][4];
#pragma unroll
  for (int i = 0; i < 2; ++i)
#pragma unroll
    for (int b = 0; b < 4; ++b) acc[i][b] = f32x16_t{};

  issue(0, 0);
  for (int ks = 0; ks < nks; ++ks) {
    __builtin_amdgcn_s_waitcnt(0x0f70);  // vmcnt(0): this wave's loads of slab ks are in LDS
    __syncthreads();                     // ... and every wave's; slab ks - 1 fully consumed
    if (ks + 1 < nks) issue(ks + 1, (ks + 1) & 1);
    const unsigned char *st = smem + (ks & 1) * kT8Stage;
    u32x4_t fa[2][2], fb[2][4];
    auto fread = [&](int kk, int slot) {
      const int c = 2 * kk + lh;
      fa[slot][0] = *reinterpret_cast<const u32x4_t *>(st + t8_off(wt0 + li, c));
      fa[slot][1] = *reinterpret_cast<const u32x4_t *>(st + t8_off(wt1 + li, c));
#pragma unroll
      for (int b = 0; b < 4; ++b)
        fb[slot][b] = *reinterpret_cast<const u32x4_t *>(st + t8_off(kT8W + b * 32 + li, c));
    };
    fread(0, 0);
#pragma unroll
    for (int kk = 0; kk < 4; ++kk) {
      if (kk + 1 < 4) fread(kk + 1, (kk + 1) & 1);
#pragma unroll
      for (int b = 0; b < 4; ++b) {
        mma32(acc[0][b], fa[kk & 1][0], fb[kk & 1][b]);
        mma32(acc[1][b], fa[kk & 1][1], fb[kk & 1][b]);
      }
    }
  }
  tile_finish<GATE_UP, false, kT8W>(a, acc, blk, e, n0, wt0, wt1, li, lh);
}

// LoRA shrink for 128-row blocks: z[pos][c] = X[pos] . A[a][e][c] for the
// rows of one LoRA tile, X = x by token (gate_up) or h by position (down).
// Two workgroups per tile, one per 64-row half of the block (a half without
// rows of the tile exits at once): A (r <= 64 rows, padded to 64) and the
// half's token rows are staged through LDS like the GEMM above; wave w
// takes token tile w % 2 of the half against A rows 32 (w / 2) .. +31.
// Rows outside the tile's run load zeros.  A workgroup covers the whole
// contraction, so z is final (no partial sums).
template <bool FROM_H, int BK, bool EVEN_K>
__global__ __launch_bounds__(kTThreads) void k_tiled_shrink(GemmArgs a) {
  using L = Lds<BK>;
  constexpr int kAR = 64;  // A rows staged (r <= 64)
  constexpr int kABytes = kAR * BK * 2, kStage = kABytes + L::kBBytes;
  __shared__ __align__(16) unsigned char smem[2 * kStage];
  const Shape &s = a.s;
  const int tile = blockIdx.x;
  if (tile >= a.al.counts[2]) return;
  const int tid = threadIdx.x, lane = tid & (kWave - 1), wave = tid / kWave;
  // the first tile also clears the zero row that masked expand lanes read
  if (a.z2 && tile == 0 && blockIdx.y == 0 && tid < 8)
    reinterpret_cast<u32x4_t *>(a.zero_row)[tid] = u32x4_t{0, 0, 0, 0};
  const int4 tl = reinterpret_cast<const int4 *>(a.al.tiles)[tile];
  const int blk = tl.x, ad = tl.y, lo = tl.z, n = tl.w;
  // workgroup y takes the tile's rows in block rows r0 .. r0 + kSR - 1
  constexpr int kSR = kTM / 2;
  const int r0 = kSR * blockIdx.y;
  if (lo >= r0 + kSR || lo + n <= r0) return;
  const int e = a.al.block_expert[blk];
  const int li = lane & 31, lh = lane >> 5;
  const int r = s.r;
  const int K = FROM_H ? s.I : s.H;

  constexpr int kRowStep = kTThreads / L::kCpr;
  constexpr int kALoads = kAR / kRowStep, kBLoads = kSR / kRowStep;
  const int lc = tid % L::kCpr, lr = tid / L::kCpr;
  const uint16_t *arow[kALoads];
#pragma unroll
  for (int j = 0; j < kALoads; ++j)
    arow[j] = static_cast<const uint16_t *>(a.A) +
              (((size_t)ad * s.E + e) * r + min(lr + j * kRowStep, r - 1)) * K;
  const uint16_t *brow[kBLoads];
  bool bok[kBLoads];
#pragma unroll
  for (int j = 0; j < kBLoads; ++j) {
    const int rr = r0 + lr + j * kRowStep;
    const int pos = blk * kTM + rr;
    bok[j] = rr >= lo && rr < lo + n;
    if (FROM_H) {
      brow[j] = static_cast<const uint16_t *>(a.h) + (size_t)pos * s.I;
    } else {
      const int p = bok[j] ? a.al.sorted_rows[pos] : 0;
      brow[j] = static_cast<const uint16_t *>(a.x) + (size_t)(p / s.k) * s.H;
    }
  }
  u32x4_t ra[kALoads], rb[kBLoads];
  auto gload = [&](int ks) {
    const int k = ks * BK + lc * 8;
#pragma unroll
    for (int j = 0; j < kALoads; ++j)
      ra[j] = EVEN_K ? load_chunk(arow[j], k) : load_chunk_any<uint16_t, true>(arow[j], k, K);
#pragma unroll
    for (int j = 0; j < kBLoads; ++j) {
      rb[j] = u32x4_t{0, 0, 0, 0};
      if (bok[j]) rb[j] = EVEN_K ? load_chunk(brow[j], k) : load_chunk_any<uint16_t, true>(brow[j], k, K);
    }
  };
  auto lstore = [&](int buf) {
    unsigned char *sa = smem + buf * kStage, *sb = sa + kABytes;
#pragma unroll
    for (int j = 0; j < kALoads; ++j)
      *reinterpret_cast<u32x4_t *>(sa + L::off(lr + j * kRowStep, lc)) = ra[j];
#pragma unroll
    for (int j = 0; j < kBLoads; ++j)
      *reinterpret_cast<u32x4_t *>(sb + L::off(lr + j * kRowStep, lc)) = rb[j];
  };

  // wave: token tile ti (32 rows of the half) against A rows 32 ai .. +31
  const int ti = wave & 1, ai = wave >> 1;
  f32x16_t acc = f32x16_t{};
  const int nks = (K + BK - 1) / BK;
  gload(0);
  lstore(0);
  __syncthreads();
  for (int ks = 0; ks < nks; ++ks) {
    const int buf = ks & 1;
    if (ks + 1 < nks) gload(ks + 1);
    const unsigned char *sa = smem + buf * kStage, *sb = sa + kABytes;
#pragma unroll
    for (int kk = 0; kk < BK / 16; ++kk) {
      const int c = 2 * kk + lh;
      const u32x4_t a0 = *reinterpret_cast<const u32x4_t *>(sa + L::off(32 * ai + li, c));
      const u32x4_t bt = *reinterpret_cast<const u32x4_t *>(sb + L::off(32 * ti + li, c));
      mma32(acc, a0, bt);
    }
    if (ks + 1 < nks) lstore(buf ^ 1);
    __syncthreads();
  }
  // lane: token row r0 + 32 ti + li; A rows 32 ai + 8 (v/4) + 4 lh + v%4
  const int local = r0 + 32 * ti + li;
  if (a.z2) {
    // bf16 rows (hi | lo): hi = bf16(z), lo = bf16(z - hi)
    if (local < lo || local >= lo + n) return;
    uint16_t *zrow = reinterpret_cast<uint16_t *>(a.z_out) + ((size_t)blk * kTM + local) * 2 * r;
#pragma unroll
    for (int g = 0; g < 4; ++g) {
      const int c = 32 * ai + 8 * g + 4 * lh;
      if (c >= r) continue;  // r is a multiple of 32 here
      uint16_t hi[4], lo4[4];
#pragma unroll
      for (int v = 0; v < 4; ++v) {
        const float zv = acc[4 * g + v];
        hi[v] = f32_to_bf16(zv);
        lo4[v] = f32_to_bf16(zv - bf16_to_f32(hi[v]));
      }
      *reinterpret_cast<uint2 *>(zrow + c) = __builtin_bit_cast(uint2, hi);
      *reinterpret_cast<uint2 *>(zrow + r + c) = __builtin_bit_cast(uint2, lo4);
    }
    return;
  }
  if (local < lo || local >= lo + n) return;
  float *zrow = a.z_out + ((size_t)blk * kTM + local) * r;
#pragma unroll
  for (int g = 0; g < 4; ++g) {
    const int c = 32 * ai + 8 * g + 4 * lh;
    if (c + 3 < r) {
      *reinterpret_cast<float4 *>(zrow + c) =
          make_float4(acc[4 * g], acc[4 * g + 1], acc[4 * g + 2], acc[4 * g + 3]);
    } else {
      for (int v = 0; v < 4; ++v)
        if (c + v < r) zrow[c + v] = acc[4 * g + v];
    }
  }
}

template <bool GATE_UP, int BK, bool EVEN_K, bool LORA>
hipError_t go_tiled(const GemmArgs &a, hipStream_t st) {
  const int cols = GATE_UP ? kTW / 2 : kTW;
  const int ntn = ((GATE_UP ? a.s.I : a.s.H) + cols - 1) / cols;
  const size_t lds = 2 * (size_t)Lds<BK>::kStage;
  auto kern = k_tiled<GATE_UP, BK, EVEN_K, LORA>;
  hipError_t err = hipFuncSetAttribute(reinterpret_cast<const void *>(kern),
                                       hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
  if (err != hipSuccess) return err;
  return launch_kernel(kern, dim3(round_up8(ntn * a.s.nblk)), dim3(kTThreads), lds, st, a);
}

template <bool GATE_UP, bool LORA>
hipError_t go_tiled8(const GemmArgs &a, hipStream_t st) {
  const int cols = GATE_UP ? kT8W / 2 : kT8W;
  const int ntn = ((GATE_UP ? a.s.I : a.s.H) + cols - 1) / cols;
  auto kern = k_tiled8<GATE_UP, LORA>;
  hipError_t err = hipFuncSetAttribute(reinterpret_cast<const void *>(kern),
                                       hipFuncAttributeMaxDynamicSharedMemorySize, kT8Lds);
  if (err != hipSuccess) return err;
  return launch_kernel(kern, dim3(round_up8(ntn * a.s.nblk)), dim3(kT8Threads), kT8Lds, st, a);
}

template <bool GATE_UP, int BK>
hipError_t pick_tiled(const GemmArgs &a, bool even_k, bool lora, hipStream_t st) {
  if (even_k) return lora ? go_tiled<GATE_UP, BK, true, true>(a, st) : go_tiled<GATE_UP, BK, true, false>(a, st);
  return lora ? go_tiled<GATE_UP, BK, false, true>(a, st) : go_tiled<GATE_UP, BK, false, false>(a, st);
}

}  // namespace

hipError_t launch_tiled_shrink(const GemmArgs &a, bool from_h, hipStream_t st) {
  if (a.s.max_tiles == 0) return hipSuccess;
  if (a.s.BM != kTM || a.s.r > 64 || a.s.r % 8 != 0 || a.split != 1) return hipErrorInvalidValue;
  const int K = from_h ? a.s.I : a.s.H;
  const bool even = K % 64 == 0;
#define MOELORA_TS(FH, EV) \
  return launch_kernel(k_tiled_shrink<FH, 64, EV>, dim3(a.s.max_tiles, 2), dim3(kTThreads), 0, st, a)
  if (from_h) {
    if (even) MOELORA_TS(true, true);
    MOELORA_TS(true, false);
  }
  if (even) MOELORA_TS(false, true);
  MOELORA_TS(false, false);
#undef MOELORA_TS
}

hipError_t launch_tiled(const GemmArgs &a, bool gate_up, const GemmVariant &v, hipStream_t st) {
  if (a.s.nblk == 0) return hipSuccess;
  if (!v.bf16 || !v.vec || a.s.BM != kTM) return hipErrorInvalidValue;
  const int K = gate_up ? a.s.H : a.s.I;
  if (K % 64 == 0 && (!v.lora || a.z2))
    return gate_up ? (v.lora ? go_tiled8<true, true>(a, st) : go_tiled8<true, false>(a, st))
                   : (v.lora ? go_tiled8<false, true>(a, st) : go_tiled8<false, false>(a, st));
  return gate_up ? pick_tiled<true, 32>(a, K % 32 == 0, v.lora, st)
                 : pick_tiled<false, 32>(a, K % 32 == 0, v.lora, st);
}

}  // namespace moelora
