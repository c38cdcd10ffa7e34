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
// first item), and each weight element is loaded once: in bf16 with a
// contraction that is a multiple of 64 through a small per-wave LDS ring
// filled with whole-line loads (contract_dma), otherwise straight into the
// register that feeds the MFMA (contract_groups).  The contraction index
// inside a chunk is never interpreted: A and B chunks of a lane always cover
// the same indices, and both paths feed the MFMAs the same indices in the
// same order.
//
// Work decomposition.  gate_up and down: one workgroup per (output columns
// of its waves, BM-row block, BM = 16, 32 or 64); the expert's weight tile
// streams through once per block, and blocks of the same expert sit on the
// same XCD so a second block finds the tile in L2.  Small workgroups (one
// to four waves) keep thousands of them in flight, which is what the weight
// stream of a decode step needs.  A gate_up wave holds 16 gate and the 16
// matching up rows; a down wave 16 rows, or two 16-row tiles that share
// each h fragment (32-row blocks).  Shrink: one workgroup per LoRA tile; its waves split
// the (16-row group of A, token group, contraction) work, and when the
// contraction is split the partial sums meet in LDS and are added in a
// fixed order, so results never depend on scheduling.
#include "common.h"
#include "kernels.h"
#include "rowlora.h"

namespace moelora {

namespace {

template <typename DT, bool VEC>
__device__ __forceinline__ u32x4_t ld(const DT *row, int k, int len) {
  if (VEC) return load_chunk(row, k);
  return load_chunk_masked(row, k, len);
}

// acc[tg] += W_rows . X_rows^T over the whole contraction for NG token
// groups.  Branch-free: every lane loads its operands unconditionally (a
// padding row's x pointer aims at a valid row and its output column is never
// written), which keeps the compiler's load counters exact so the two
// register sets below really overlap.
template <typename DT, int NG, int U, bool VEC, bool EVEN_K, bool TWO>
__device__ __forceinline__ void contract_groups(const DT *w0, const DT *w1, const DT *const *xr,
                                                int K, int kg, f32x4_t *acc0, f32x4_t *acc1) {
  using M = Mma<DT>;
  constexpr int EPC = Elem<DT>::kPerChunk;
  constexpr int KS = M::kK;
  const int nfull = K / KS;
  // Groups of U contraction steps in two register sets: the loads of group
  // g + 1 are issued before the MFMAs of group g, so the weight stream never
  // drains while a group waits for its slowest load.
  struct Group {
    u32x4_t a0[U], a1[U], b[U][NG];
  };
  auto load = [&](Group &g, int grp) {
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int k = (grp * U + u) * KS + kg * EPC;
      g.a0[u] = ld<DT, VEC>(w0, k, K);
      if (TWO) g.a1[u] = ld<DT, VEC>(w1, k, K);
#pragma unroll
      for (int tg = 0; tg < NG; ++tg) g.b[u][tg] = ld<DT, VEC>(xr[tg], k, K);
    }
  };
  auto compute = [&](const Group &g) {
#pragma unroll
    for (int u = 0; u < U; ++u)
#pragma unroll
      for (int tg = 0; tg < NG; ++tg) {
        M::step(acc0[tg], g.a0[u], g.b[u][tg]);
        if (TWO) M::step(acc1[tg], g.a1[u], g.b[u][tg]);
      }
  };
  const int ngroups = nfull / U;
  Group ga, gb;
  if (ngroups > 0) load(ga, 0);
  // The loop body issues its loads unconditionally (the last pass reloads
  // the final group, an L2 hit): a conditional load would leave the
  // compiler unsure how many younger loads are outstanding, and it would
  // then wait for all of them before the current group's MFMAs.
  int grp = 0;
  for (; grp + 2 <= ngroups; grp += 2) {
    load(gb, grp + 1);
    compute(ga);
    load(ga, min(grp + 2, ngroups - 1));
    compute(gb);
  }
  if (grp < ngroups) compute(ga);  // odd group count: the last one is in ga
  for (int st = ngroups * U; st < nfull; ++st) {
    const int k = st * KS + kg * EPC;
    const u32x4_t a0 = ld<DT, VEC>(w0, k, K);
    const u32x4_t a1 = TWO ? ld<DT, VEC>(w1, k, K) : a0;
#pragma unroll
    for (int tg = 0; tg < NG; ++tg) {
      const u32x4_t b = ld<DT, VEC>(xr[tg], k, K);
      M::step(acc0[tg], a0, b);
      if (TWO) M::step(acc1[tg], a1, b);
    }
  }
  if (!EVEN_K) {  // the masked tail step: K is not a multiple of the step
    const int k = nfull * KS + kg * EPC;
    const u32x4_t a0 = load_chunk_any<DT, VEC>(w0, k, K);
    const u32x4_t a1 = TWO ? load_chunk_any<DT, VEC>(w1, k, K) : a0;
#pragma unroll
    for (int tg = 0; tg < NG; ++tg) {
      const u32x4_t b = load_chunk_any<DT, VEC>(xr[tg], k, K);
      M::step(acc0[tg], a0, b);
      if (TWO) M::step(acc1[tg], a1, b);
    }
  }
}

// The block's contraction over its ntg leading token groups (the rest hold
// only padding and are skipped): one branch-free instance per group count.
template <typename DT, int TG, int U, bool VEC, bool EVEN_K, bool TWO>
__device__ __forceinline__ void contract(const DT *w0, const DT *w1, const DT *const *xr, int ntg,
                                         int K, int kg, f32x4_t *acc0, f32x4_t *acc1) {
  if (TG >= 4 && ntg > 2)
    contract_groups<DT, TG, U, VEC, EVEN_K, TWO>(w0, w1, xr, K, kg, acc0, acc1);
  else if (TG >= 2 && ntg > 1)
    contract_groups<DT, (TG >= 2 ? 2 : 1), U, VEC, EVEN_K, TWO>(w0, w1, xr, K, kg, acc0, acc1);
  else
    contract_groups<DT, 1, U, VEC, EVEN_K, TWO>(w0, w1, xr, K, kg, acc0, acc1);
}

// Weight stream through LDS (bf16, contraction a multiple of 64).  A wave's
// NW 16-row weight tiles are fetched in 64-wide slabs: slab j of tile t is
// 16 rows x 128 bytes, brought by two global_load_lds_dwordx4 of 8 whole
// rows each (lane l: row l / 8, one 16-byte chunk), so every load
// instruction covers whole 128-byte lines -- the register path above has a
// lane per (row, chunk of a 64-byte half line) and streams slower.  Slabs go
// round a per-wave ring of S >= 2 slots in LDS.  Step j first waits until
// the LDS reads of step j - 1 have returned (they read the slot refilled
// now), then issues the P = 2 NW + 2 NG loads of the step: slab j + S - 1
// into its slot and the tokens of slab j + 1 into registers; then it waits
// with vmcnt(P), i.e. for everything but the step's own P loads, and
// computes slab j.  Every load of slab j was issued before this step's
// loads (at step j - S + 1, or before the loop), and vector-memory loads,
// direct-to-LDS ones included, retire in issue order, so the wait has
// landed slab j in LDS and its tokens in registers (with S >= 3 it has also
// landed slabs j + 1 .. j + S - 2).  Compiler barriers keep each step's
// loads on their side of its waits, and each slab issues exactly P vector
// loads (past the end the last slab is fetched again into a free slot), so
// the fixed count holds; the kernels use no scratch memory, whose reloads
// would be vector loads too.
// The MFMA operand of lane l (row l % 16, chunk l / 16 of a 32-wide step) is then
// one ds_read_b128.  Chunk c of tile row r sits at chunk c ^ (r % 8) of its
// LDS row, so the 16 rows read at one chunk spread over distinct banks.
// Tokens (L2-resident, shared by every workgroup of the block) are loaded
// straight into registers, one slab ahead.
// Weight loads are marked non-temporal: each line is read once.  rot
// (0 <= rot < K / 64) starts the walk at slab rot and wraps around: with
// row strides that are multiples of 4 KB, workgroups that walk the same
// slab columns at once stream ~13 % slower than staggered ones.
// s_waitcnt immediates (gfx9 encoding: vmcnt bits 3:0 and 15:14, expcnt
// 6:4, lgkmcnt 11:8; an all-ones field waits for nothing).
constexpr int waitcnt_vm(int n) { return 0x0f70 | (n & 15) | ((n >> 4) << 14); }
constexpr int waitcnt_vm_lgkm0(int n) { return 0x0070 | (n & 15) | ((n >> 4) << 14); }
constexpr int kWaitLgkm0 = 0xc07f;  // lgkmcnt(0): every LDS read has returned
template <int NG, int NW, int S>
__device__ __forceinline__ void contract_dma(const uint16_t *const *dsrc,
                                             const uint16_t *const *xr, int K, int kg, int ri,
                                             int rot, unsigned char *ring, f32x4_t *acc0,
                                             f32x4_t *acc1) {
  using M = Mma<uint16_t>;
  static_assert(S >= 2, "a slot is refilled while another is read");
  constexpr int kSlot = NW * 2048;
  constexpr int kPer = 2 * NW + 2 * NG;    // vector loads issued per step
  static_assert(kPer < 64, "vmcnt immediate");
  constexpr int kWait = waitcnt_vm(kPer);  // all but the step's own loads
  const int nsl = K / 64;
  auto slab = [&](int j) { return j + rot >= nsl ? j + rot - nsl : j + rot; };
  auto dma = [&](int j, int p) {
    j = slab(j);
    unsigned char *d = ring + p * kSlot;
#pragma unroll
    for (int t = 0; t < NW; ++t)
#pragma unroll
      for (int i = 0; i < 2; ++i)
        __builtin_amdgcn_global_load_lds(dsrc[2 * t + i] + 64 * j,
                                         (__attribute__((address_space(3))) void *)(d + t * 2048 + i * 1024),
                                         16, 0, kCpolNonTemporal);
  };
  struct Tok {
    u32x4_t b[2][NG];
  };
  auto tload = [&](Tok &tk, int j) {
    j = slab(j);
#pragma unroll
    for (int h = 0; h < 2; ++h)
#pragma unroll
      for (int g = 0; g < NG; ++g) tk.b[h][g] = load_chunk(xr[g], 64 * j + 32 * h + 8 * kg);
  };
  auto compute = [&](int p, const Tok &tk) {
    const unsigned char *d = ring + p * kSlot + ri * 128;
#pragma unroll
    for (int h = 0; h < 2; ++h) {
      const int c = ((4 * h + kg) ^ (ri & 7)) << 4;
      const u32x4_t a0 = *reinterpret_cast<const u32x4_t *>(d + c);
      const u32x4_t a1 = NW == 2 ? *reinterpret_cast<const u32x4_t *>(d + 2048 + c) : a0;
#pragma unroll
      for (int g = 0; g < NG; ++g) {
        M::step(acc0[g], a0, tk.b[h][g]);
        if (NW == 2) M::step(acc1[g], a1, tk.b[h][g]);
      }
    }
  };
#pragma unroll
  for (int j = 0; j < S - 1; ++j) dma(min(j, nsl - 1), j);
  // one slab: fetch slab j + S - 1 and the tokens of slab j + 1, then the
  // MFMAs of slab j once it and its tokens (tk) have arrived
  auto step = [&](int j, const Tok &tk, Tok &tn) {
    asm volatile("" ::: "memory");
    __builtin_amdgcn_s_waitcnt(kWaitLgkm0);  // slot (j + S - 1) % S has been read out
    asm volatile("" ::: "memory");
    dma(min(j + S - 1, nsl - 1), (j + S - 1) % S);
    tload(tn, min(j + 1, nsl - 1));
    asm volatile("" ::: "memory");
    __builtin_amdgcn_s_waitcnt(kWait);
    asm volatile("" ::: "memory");
    compute(j % S, tk);
  };
  Tok ta, tb;
  tload(ta, 0);
  int j = 0;
  for (; j + 2 <= nsl; j += 2) {
    step(j, ta, tb);
    step(j + 1, tb, ta);
  }
  if (j < nsl) step(j, ta, tb);
  // vmcnt(0): no load of the ring may land after the wave leaves it
  __builtin_amdgcn_s_waitcnt(0x0f70);
}

// contract_dma over the block's ntg leading token groups.
template <int TG, int NW, int S>
__device__ __forceinline__ void contract_dma_groups(const uint16_t *const *dsrc,
                                                    const uint16_t *const *xr, int ntg, int K, int kg,
                                                    int ri, int rot, unsigned char *ring,
                                                    f32x4_t *acc0, f32x4_t *acc1) {
  if (TG >= 4 && ntg > 2)
    contract_dma<TG, NW, S>(dsrc, xr, K, kg, ri, rot, ring, acc0, acc1);
  else if (TG >= 2 && ntg > 1)
    contract_dma<(TG >= 2 ? 2 : 1), NW, S>(dsrc, xr, K, kg, ri, rot, ring, acc0, acc1);
  else
    contract_dma<1, NW, S>(dsrc, xr, K, kg, ri, rot, ring, acc0, acc1);
}

// Shared-token variant of contract_dma for workgroups of kShareWaves waves
// that compute the same block against different weight rows: the block's
// token rows go through one LDS ring of the workgroup instead of every
// wave's registers, fetched with whole-line loads (global_load_lds_dwordx4
// of 8 rows x 128 bytes, the chunk swizzle of the weight tiles) and each
// fetched once for all the waves.  The 2 NG token loads of a slab are dealt
// round the waves (kTI per wave; with more waves than loads a load is issued
// twice, writing the same bytes).  Step j waits until the wave's own loads
// of slab j have landed (vmcnt leaves only the loads of the S - 2 younger
// slabs in flight) and its LDS reads of slab j - 1 have returned (lgkmcnt 0),
// then meets the other waves at a workgroup barrier: after it, every wave's
// share of slab j is in LDS and nobody reads slab j - 1 any more, so its
// slots are refilled with slab j + S - 1, and slabs j + 1 .. j + S - 1 are
// in flight while slab j is computed.  tok_row[row] is the token row of
// block row row (0 <= row < 16 NG), tbase + tok_row * ld the start of its
// contraction range.  Every wave of the workgroup must call this with the
// same K, rot and NG (the barriers are counted).
// One whole-line DMA: 64 lanes x 16 bytes from src (per lane) to lds (per
// wave; lane l's bytes land at lds + 16 l).
__device__ __forceinline__ void dma16(const uint16_t *src, unsigned char *lds, bool nontemporal) {
  if (nontemporal)
    __builtin_amdgcn_global_load_lds(src, (__attribute__((address_space(3))) void *)lds, 16, 0,
                                     kCpolNonTemporal);
  else
    __builtin_amdgcn_global_load_lds(src, (__attribute__((address_space(3))) void *)lds, 16, 0, 0);
}
__device__ __forceinline__ void dma16_bytes(const uint8_t *src, unsigned char *lds) {
  __builtin_amdgcn_global_load_lds(src, (__attribute__((address_space(3))) void *)lds, 16, 0,
                                   kCpolNonTemporal);
}
template <int NG, int NW, int S>
__device__ __forceinline__ void contract_shared(const uint16_t *const *dsrc, const uint16_t *tbase,
                                                size_t ld, const int *tok_row, int K, int kg,
                                                int ri, int wave, int rot, unsigned char *tring,
                                                int tslot, unsigned char *wring, f32x4_t *acc0,
                                                f32x4_t *acc1) {
  using M = Mma<uint16_t>;
  constexpr int kTI = (2 * NG + kShareWaves - 1) / kShareWaves;  // token loads per wave
  constexpr int kPer = 2 * NW + kTI;                              // loads per slab
  constexpr int kYoung = (S - 2) * kPer;  // loads of the slabs issued after slab j
  static_assert(S >= 2 && kYoung < 64, "vmcnt immediate");
  constexpr int kWait = waitcnt_vm_lgkm0(kYoung);
  const int lane = threadIdx.x & (kWave - 1);
  const uint16_t *tsrc[kTI];
  int tq[kTI];
#pragma unroll
  for (int c = 0; c < kTI; ++c) {
    const int q = (wave + c * kShareWaves) % (2 * NG);
    const int row = 8 * q + (lane >> 3);
    tq[c] = q;
    tsrc[c] = tbase + (size_t)tok_row[row] * ld + 8 * ((lane & 7) ^ (lane >> 3));
  }
  const int nsl = K / 64;
  auto slab = [&](int j) { return j + rot >= nsl ? j + rot - nsl : j + rot; };
  auto issue = [&](int j, int p) {
    j = slab(j);
    unsigned char *d = wring + p * NW * 2048;
#pragma unroll
    for (int t = 0; t < NW; ++t)
#pragma unroll
      for (int i = 0; i < 2; ++i) dma16(dsrc[2 * t + i] + 64 * j, d + t * 2048 + i * 1024, true);
    unsigned char *td = tring + p * tslot;
#pragma unroll
    for (int c = 0; c < kTI; ++c) dma16(tsrc[c] + 64 * j, td + tq[c] * 1024, false);
  };
  auto compute = [&](int p) {
    const unsigned char *d = wring + p * NW * 2048 + ri * 128;
    const unsigned char *td = tring + p * tslot + ri * 128;
#pragma unroll
    for (int h = 0; h < 2; ++h) {
      const int c = ((4 * h + kg) ^ (ri & 7)) << 4;
      const u32x4_t a0 = *reinterpret_cast<const u32x4_t *>(d + c);
      const u32x4_t a1 = NW == 2 ? *reinterpret_cast<const u32x4_t *>(d + 2048 + c) : a0;
#pragma unroll
      for (int g = 0; g < NG; ++g) {
        const u32x4_t b = *reinterpret_cast<const u32x4_t *>(td + g * 2048 + c);
        M::step(acc0[g], a0, b);
        if (NW == 2) M::step(acc1[g], a1, b);
      }
    }
  };
#pragma unroll
  for (int j = 0; j < S - 1; ++j) issue(min(j, nsl - 1), j);
  for (int j = 0; j < nsl; ++j) {
    asm volatile("" ::: "memory");
    __builtin_amdgcn_s_waitcnt(kWait);
    asm volatile("" ::: "memory");
    __builtin_amdgcn_s_barrier();
    asm volatile("" ::: "memory");
    issue(min(j + S - 1, nsl - 1), (j + S - 1) % S);
    compute(j % S);
  }
  // vmcnt(0): no load of the rings may land after the wave leaves them
  __builtin_amdgcn_s_waitcnt(0x0f70);
}

// contract_shared over the block's ntg leading token groups.
template <int TG, int NW, int S>
__device__ __forceinline__ void contract_shared_groups(const uint16_t *const *dsrc,
                                                       const uint16_t *tbase, size_t ld,
                                                       const int *tok_row, int ntg, int K, int kg,
                                                       int ri, int wave, int rot,
                                                       unsigned char *tring, unsigned char *wring,
                                                       f32x4_t *acc0, f32x4_t *acc1) {
  constexpr int tslot = TG * 2048;
  if (TG >= 4 && ntg > 2)
    contract_shared<TG, NW, S>(dsrc, tbase, ld, tok_row, K, kg, ri, wave, rot, tring, tslot, wring,
                               acc0, acc1);
  else if (TG >= 2 && ntg > 1)
    contract_shared<(TG >= 2 ? 2 : 1), NW, S>(dsrc, tbase, ld, tok_row, K, kg, ri, wave, rot, tring,
                                              tslot, wring, acc0, acc1);
  else
    contract_shared<1, NW, S>(dsrc, tbase, ld, tok_row, K, kg, ri, wave, rot, tring, tslot, wring,
                              acc0, acc1);
}
// E4M3 weight stream (contract_dma8 / contract_shared8: the two ring forms
// above with one-byte base weights and one scale per weight row).  A slab
// is 128 contraction elements, so a 16-row weight tile is again 16 rows x
// 128 bytes (whole lines, the same two global_load_lds_dwordx4 per tile and
// the same slot size and chunk swizzle); a contraction that is an odd
// multiple of 64 ends with a 64-wide tail slab whose upper chunks are
// fetched from the lower ones (a valid address; those bytes are not used).
// Lane (ri, kg) reads chunks kg and 4 + kg of row ri (16 codes each) and
// covers, at k-step h = 0..3, contraction indices [16 c + 8 (h & 1), +8)
// with c = kg + 4 (h >> 1) -- four lanes groups x 8 = 32 indices per step,
// all 128 over the slab; its tokens are loaded for the same indices.  The
// codes become bf16 operands in registers (e4m3x8_to_bf16, exact); the row
// scales are applied by the caller after the contraction.  Loads per step:
// 2 NW weight DMAs + 4 NG token loads (register tokens) or 2 NW + NG
// (shared tokens), with the wait arithmetic of the bf16 forms.

// Slab index of step j for a walk starting at rot (no rotation with a tail).
__device__ __forceinline__ int slab_of(int j, int rot, int nsl) {
  return j + rot >= nsl ? j + rot - nsl : j + rot;
}

template <int NG, int NW, int S>
__device__ __forceinline__ void contract_dma8(const uint8_t *const *wrow, int coff, int coff_tail,
                                              const uint16_t *const *xr, int K, int kg, int ri,
                                              int rot, unsigned char *ring, f32x4_t *acc0,
                                              f32x4_t *acc1) {
  using M = Mma<uint16_t>;
  static_assert(S >= 2, "a slot is refilled while another is read");
  constexpr int kSlot = NW * 2048;
  constexpr int kPer = 2 * NW + 4 * NG;    // vector loads issued per step
  static_assert(kPer < 64, "vmcnt immediate");
  constexpr int kWait = waitcnt_vm(kPer);
  const int nsl = (K + 127) / 128;
  const bool tail = K % 128 != 0;           // the last slab holds 64 elements
  if (tail) rot = 0;
  auto dma = [&](int j, int p) {
    j = slab_of(j, rot, nsl);
    const int off = 128 * j + (tail && j == nsl - 1 ? coff_tail : coff);
    unsigned char *d = ring + p * kSlot;
#pragma unroll
    for (int t = 0; t < NW; ++t)
#pragma unroll
      for (int i = 0; i < 2; ++i)
        __builtin_amdgcn_global_load_lds(wrow[2 * t + i] + off,
                                         (__attribute__((address_space(3))) void *)(d + t * 2048 + i * 1024),
                                         16, 0, kCpolNonTemporal);
  };
  struct Tok {
    u32x4_t b[4][NG];
  };
  auto tload = [&](Tok &tk, int j) {
    j = slab_of(j, rot, nsl);
    const bool tj = tail && j == nsl - 1;
#pragma unroll
    for (int h = 0; h < 4; ++h) {
      const int c = kg + (h >= 2 && !tj ? 4 : 0);
#pragma unroll
      for (int g = 0; g < NG; ++g) tk.b[h][g] = load_chunk(xr[g], 128 * j + 16 * c + 8 * (h & 1));
    }
  };
  auto compute = [&](int p, const Tok &tk, bool last_tail) {
    const unsigned char *d = ring + p * kSlot + ri * 128;
    const int clo = (kg ^ (ri & 7)) << 4, chi = ((4 + kg) ^ (ri & 7)) << 4;
#pragma unroll
    for (int t = 0; t < NW; ++t) {
      f32x4_t *acc = t == 0 ? acc0 : acc1;
      const u32x4_t lo = *reinterpret_cast<const u32x4_t *>(d + t * 2048 + clo);
      const u32x4_t a0 = e4m3x8_to_bf16(lo[0], lo[1]), a1 = e4m3x8_to_bf16(lo[2], lo[3]);
#pragma unroll
      for (int g = 0; g < NG; ++g) {
        M::step(acc[g], a0, tk.b[0][g]);
        M::step(acc[g], a1, tk.b[1][g]);
      }
      if (!last_tail) {
        const u32x4_t hi = *reinterpret_cast<const u32x4_t *>(d + t * 2048 + chi);
        const u32x4_t a2 = e4m3x8_to_bf16(hi[0], hi[1]), a3 = e4m3x8_to_bf16(hi[2], hi[3]);
#pragma unroll
        for (int g = 0; g < NG; ++g) {
          M::step(acc[g], a2, tk.b[2][g]);
          M::step(acc[g], a3, tk.b[3][g]);
        }
      }
    }
  };
#pragma unroll
  for (int j = 0; j < S - 1; ++j) dma(min(j, nsl - 1), j);
  auto step = [&](int j, const Tok &tk, Tok &tn, bool last_tail) {
    asm volatile("" ::: "memory");
    __builtin_amdgcn_s_waitcnt(kWaitLgkm0);  // slot (j + S - 1) % S has been read out
    asm volatile("" ::: "memory");
    dma(min(j + S - 1, nsl - 1), (j + S - 1) % S);
    tload(tn, min(j + 1, nsl - 1));
    asm volatile("" ::: "memory");
    __builtin_amdgcn_s_waitcnt(kWait);
    asm volatile("" ::: "memory");
    compute(j % S, tk, last_tail);
  };
  Tok ta, tb;
  tload(ta, 0);
  // every step but the last one in pairs; the last step may be the tail
  int j = 0;
  for (; j + 2 <= nsl - 1; j += 2) {
    step(j, ta, tb, false);
    step(j + 1, tb, ta, false);
  }
  if (j < nsl - 1) {
    step(j, ta, tb, false);
    step(j + 1, tb, ta, tail);
  } else {
    step(j, ta, tb, tail);
  }
  __builtin_amdgcn_s_waitcnt(0x0f70);  // vmcnt(0): no load of the ring lands after the wave leaves it
}

template <int TG, int NW, int S>
__device__ __forceinline__ void contract_dma8_groups(const uint8_t *const *wrow, int coff,
                                                     int coff_tail, const uint16_t *const *xr,
                                                     int ntg, int K, int kg, int ri, int rot,
                                                     unsigned char *ring, f32x4_t *acc0,
                                                     f32x4_t *acc1) {
  if (TG >= 4 && ntg > 2)
    contract_dma8<TG, NW, S>(wrow, coff, coff_tail, xr, K, kg, ri, rot, ring, acc0, acc1);
  else if (TG >= 2 && ntg > 1)
    contract_dma8<(TG >= 2 ? 2 : 1), NW, S>(wrow, coff, coff_tail, xr, K, kg, ri, rot, ring, acc0,
                                            acc1);
  else
    contract_dma8<1, NW, S>(wrow, coff, coff_tail, xr, K, kg, ri, rot, ring, acc0, acc1);
}

// Shared-token form: each group's token slab (16 rows x 128 bf16 = 4 KB)
// sits in LDS as two halves of 16 rows x 128 bytes (contraction [0, 64) and
// [64, 128) of the slab), each written by two whole-line DMAs of 8 rows, so
// a slab is 4 NG token loads dealt round the waves (NG per wave).
template <int NG, int NW, int S>
__device__ __forceinline__ void contract_shared8(const uint8_t *const *wrow, int coff, int coff_tail,
                                                 const uint16_t *tbase, size_t ld,
                                                 const int *tok_row, int K, int kg, int ri,
                                                 int wave, int rot, unsigned char *tring,
                                                 int tslot, unsigned char *wring, f32x4_t *acc0,
                                                 f32x4_t *acc1) {
  using M = Mma<uint16_t>;
  constexpr int kTI = (4 * NG + kShareWaves - 1) / kShareWaves;  // token loads per wave
  constexpr int kPer = 2 * NW + kTI;                              // loads per slab
  constexpr int kYoung = (S - 2) * kPer;  // loads of the slabs issued after slab j
  static_assert(S >= 2 && kYoung < 64, "vmcnt immediate");
  constexpr int kWait = waitcnt_vm_lgkm0(kYoung);
  const int lane = threadIdx.x & (kWave - 1);
  const int nsl = (K + 127) / 128;
  const bool tail = K % 128 != 0;
  if (tail) rot = 0;
  // token load q (0 <= q < 4 NG) of a slab: group q / 4, half (q / 2) % 2,
  // rows 8 (q % 2) .. +7; lane l: row 8 (q % 2) + l / 8, source chunk
  // (l % 8) ^ (l / 8) of the half
  const uint16_t *tsrc[kTI];
  int tq[kTI];
#pragma unroll
  for (int c = 0; c < kTI; ++c) {
    const int q = (wave + c * kShareWaves) % (4 * NG);
    const int row = 16 * (q / 4) + 8 * (q % 2) + (lane >> 3);
    tq[c] = q;
    tsrc[c] = tbase + (size_t)tok_row[row] * ld + 8 * ((lane & 7) ^ (lane >> 3));
  }
  auto issue = [&](int j, int p) {
    j = slab_of(j, rot, nsl);
    const bool tj = tail && j == nsl - 1;
    const int off = 128 * j + (tj ? coff_tail : coff);
    unsigned char *d = wring + p * NW * 2048;
#pragma unroll
    for (int t = 0; t < NW; ++t)
#pragma unroll
      for (int i = 0; i < 2; ++i) dma16_bytes(wrow[2 * t + i] + off, d + t * 2048 + i * 1024);
    unsigned char *td = tring + p * tslot;
#pragma unroll
    for (int c = 0; c < kTI; ++c) {
      const int q = tq[c], half = (q >> 1) & 1;
      dma16(tsrc[c] + 128 * j + (tj ? 0 : 64 * half), td + (q >> 2) * 4096 + half * 2048 + (q & 1) * 1024,
            false);
    }
  };
  auto compute = [&](int p, bool last_tail) {
    const unsigned char *d = wring + p * NW * 2048 + ri * 128;
    const unsigned char *td = tring + p * tslot + ri * 128;
    const int clo = (kg ^ (ri & 7)) << 4, chi = ((4 + kg) ^ (ri & 7)) << 4;
    // token chunk of k-step h: element 16 c + 8 (h & 1), c = kg + 4 (h >> 1)
    // -> half h >> 1, chunk 2 kg + (h & 1) of that half
    const int t0 = ((2 * kg) ^ (ri & 7)) << 4, t1 = ((2 * kg + 1) ^ (ri & 7)) << 4;
#pragma unroll
    for (int t = 0; t < NW; ++t) {
      f32x4_t *acc = t == 0 ? acc0 : acc1;
      const u32x4_t lo = *reinterpret_cast<const u32x4_t *>(d + t * 2048 + clo);
      const u32x4_t a0 = e4m3x8_to_bf16(lo[0], lo[1]), a1 = e4m3x8_to_bf16(lo[2], lo[3]);
#pragma unroll
      for (int g = 0; g < NG; ++g) {
        M::step(acc[g], a0, *reinterpret_cast<const u32x4_t *>(td + g * 4096 + t0));
        M::step(acc[g], a1, *reinterpret_cast<const u32x4_t *>(td + g * 4096 + t1));
      }
      if (!last_tail) {
        const u32x4_t hi = *reinterpret_cast<const u32x4_t *>(d + t * 2048 + chi);
        const u32x4_t a2 = e4m3x8_to_bf16(hi[0], hi[1]), a3 = e4m3x8_to_bf16(hi[2], hi[3]);
#pragma unroll
        for (int g = 0; g < NG; ++g) {
          M::step(acc[g], a2, *reinterpret_cast<const u32x4_t *>(td + g * 4096 + 2048 + t0));
          M::step(acc[g], a3, *reinterpret_cast<const u32x4_t *>(td + g * 4096 + 2048 + t1));
        }
      }
    }
  };
#pragma unroll
  for (int j = 0; j < S - 1; ++j) issue(min(j, nsl - 1), j);
  for (int j = 0; j < nsl; ++j) {
    asm volatile("" ::: "memory");
    __builtin_amdgcn_s_waitcnt(kWait);
    asm volatile("" ::: "memory");
    __builtin_amdgcn_s_barrier();
    asm volatile("" ::: "memory");
    issue(min(j + S - 1, nsl - 1), (j + S - 1) % S);
    compute(j % S, tail && j == nsl - 1);
  }
  __builtin_amdgcn_s_waitcnt(0x0f70);  // vmcnt(0): no load of the rings lands after the wave leaves them
}

template <int TG, int NW, int S>
__device__ __forceinline__ void contract_shared8_groups(const uint8_t *const *wrow, int coff,
                                                        int coff_tail, const uint16_t *tbase,
                                                        size_t ld, const int *tok_row, int ntg,
                                                        int K, int kg, int ri, int wave, int rot,
                                                        unsigned char *tring, unsigned char *wring,
                                                        f32x4_t *acc0, f32x4_t *acc1) {
  constexpr int tslot = TG * 4096;
  if (TG >= 4 && ntg > 2)
    contract_shared8<TG, NW, S>(wrow, coff, coff_tail, tbase, ld, tok_row, K, kg, ri, wave, rot,
                                tring, tslot, wring, acc0, acc1);
  else if (TG >= 2 && ntg > 1)
    contract_shared8<(TG >= 2 ? 2 : 1), NW, S>(wrow, coff, coff_tail, tbase, ld, tok_row, K, kg, ri,
                                               wave, rot, tring, tslot, wring, acc0, acc1);
  else
    contract_shared8<1, NW, S>(wrow, coff, coff_tail, tbase, ld, tok_row, K, kg, ri, wave, rot,
                               tring, tslot, wring, acc0, acc1);
}

// The E4M3 weight rows of one DMA lane: rows 8 i + lane / 8 of each 16-row
// tile, and its chunk's byte offset within a slab (full and tail slab).
struct W8Rows {
  const uint8_t *row[4];
  int coff, coff_tail;
};

// Scales of the four weight rows an MFMA output lane holds (rows
// m + 4 kg .. +3 of a 16-row tile at m), applied to the accumulators.  They
// are loaded before the contraction (row_scales), so the epilogue does not
// wait for them; a tile past the last row reads the last valid tile's.
__device__ __forceinline__ float4 row_scales(const float *scale, int kg) {
  return *reinterpret_cast<const float4 *>(scale + 4 * kg);
}
template <int TG>
__device__ __forceinline__ void scale_rows(float4 s4, f32x4_t *acc) {
#pragma unroll
  for (int tg = 0; tg < TG; ++tg) {
    acc[tg][0] *= s4.x;
    acc[tg][1] *= s4.y;
    acc[tg][2] *= s4.z;
    acc[tg][3] *= s4.w;
  }
}

// Starting slab of a workgroup's weight walk (contract_dma): staggered over
// column tiles when a.rotate is set, else 0.  Keyed on the column tile, not
// the workgroup, so that the blocks of one expert, which stream the same
// weight rows, walk them in step and can meet in L2.
__device__ __forceinline__ int walk_start(const GemmArgs &a, int K, int col_tile) {
  return a.rotate ? (int)(((unsigned)col_tile * 7u) % (unsigned)(K / 64)) : 0;
}
// The same for the E4M3 stream's 128-wide slabs.
__device__ __forceinline__ int walk_start8(const GemmArgs &a, int K, int col_tile) {
  return a.rotate ? (int)(((unsigned)col_tile * 7u) % (unsigned)((K + 127) / 128)) : 0;
}

// z values of a lane's rows for the batched expand below: row mode, z of
// routed row prow[tg]; tile mode (one contraction split), z of sorted
// position blk * BM + tg * 16 + ri.  Neither depends on the LoRA tile, so
// they are loaded once, before the base contraction, and their latency
// hides under it, as does that of the descriptors of the expand's first
// two batches of tiles (lane u % (2 kExpandBatch) holds tile
// t0 + u % (2 kExpandBatch)).
// A padding row reads row 0 / its own unused position; its value is never
// selected.
constexpr int kExpandBatch = 8;
template <typename DT, int TG>
struct ZRows {
  float v[TG][Elem<DT>::kPerChunk];
  int4 dl0;
};

template <typename DT, bool VEC, bool ROWZ>
__device__ __forceinline__ bool expand_batched(const GemmArgs &a) {
  return VEC && a.s.r <= Mma<DT>::kK && (ROWZ || a.split == 1);
}

template <typename DT, int TG, bool ROWZ>
__device__ __forceinline__ void load_zrows(const GemmArgs &a, int blk, int t0, int t1, int kg,
                                           int ri, const int *prow, ZRows<DT, TG> &z) {
  constexpr int EPC = Elem<DT>::kPerChunk;
  const int r = a.s.r, kk = kg * EPC, kc = kk < r ? kk : 0;
  if (t1 > t0)
    z.dl0 = reinterpret_cast<const int4 *>(
        a.al.tiles)[min(t0 + (int)(threadIdx.x & (2 * kExpandBatch - 1)), t1 - 1)];
#pragma unroll
  for (int tg = 0; tg < TG; ++tg) {
    const size_t row = ROWZ ? (size_t)(prow[tg] < a.s.R ? prow[tg] : 0)
                            : (size_t)blk * 16 * TG + tg * 16 + ri;
    const float *zp = a.z + row * r + kc;
#pragma unroll
    for (int q = 0; q < EPC; q += 4) {
      const float4 v4 = *reinterpret_cast<const float4 *>(zp + q);
      z.v[tg][q] = v4.x;
      z.v[tg][q + 1] = v4.y;
      z.v[tg][q + 2] = v4.z;
      z.v[tg][q + 3] = v4.w;
    }
  }
}

// The expand of one projection, added into the base accumulators:
// acc[tg] += B_rows . z^T for the block's LoRA tiles t0 .. t1-1.  z (float)
// feeds the MFMA as a bf16 hi + lo pair (a split exact to about 2^-16) or
// as float.
template <typename DT, int TG, bool VEC, bool TWO, bool ROWZ>
__device__ __forceinline__ void expand(const GemmArgs &a, int blk, int e, int t0, int t1,
                                       const ZRows<DT, TG> &zr, const DT *Bbase, size_t b_rows,
                                       int row, size_t row_off1, int kg, int ri, const int *prow,
                                       f32x4_t *acc0, f32x4_t *acc1) {
  using M = Mma<DT>;
  constexpr int EPC = Elem<DT>::kPerChunk;
  constexpr int KS = M::kK;
  constexpr int BM = 16 * TG;
  const Shape &s = a.s;
  const int r = s.r;
  if constexpr (VEC) {
    if (expand_batched<DT, VEC, ROWZ>(a)) {
      // One contraction step per tile (r <= KS), z already in registers:
      // the descriptors and B chunks of eight tiles are loaded together,
      // then their MFMAs run in tile order.  32-row blocks of a skewed
      // many-adapter batch carry up to ~18 tiles, whose expand then ends the
      // kernel's slowest workgroups; the registers are free (the LDS ring,
      // not the register file, limits these kernels' occupancy).  Loads are
      // unconditional (a lane past the rank reads a valid address and its
      // value is zeroed).
      constexpr int TB = kExpandBatch;
      const int kk = kg * EPC, kc = kk < r ? kk : 0;
      const bool kin = kk < r;
      // z of the lane's rows split into MFMA operands once (a row outside
      // a tile takes zero, whose split is zero)
      u32x4_t zh[TG], zl[TG];
#pragma unroll
      for (int tg = 0; tg < TG; ++tg) {
        float z[EPC];
#pragma unroll
        for (int q = 0; q < EPC; ++q) z[q] = kin ? zr.v[tg][q] : 0.f;
        SplitF32<DT>::run(z, zh[tg], zl[tg]);
      }
      for (int tb = t0; tb < t1; tb += TB) {
        // The batch's descriptors in one load (lane u % TB holds tile
        // tb + u % TB), then every B load of the batch, then the MFMAs: two
        // round trips per batch.  The empty statements read the registers
        // so that each group of loads is complete before the next step;
        // otherwise the compiler interleaves per tile (a descriptor's wait
        // then also waits for the earlier tiles' B loads, and each tile's
        // loads sink down to its MFMAs past the batch's end test): one round
        // trip per tile.
        const int lu = threadIdx.x & (TB - 1);
        // the first two batches' descriptors came with z (lanes 0 .. 2 TB - 1)
        const bool pre = tb - t0 < 2 * TB;
        const int lb = tb == t0 ? 0 : pre ? TB : 0;  // lane of the batch's first tile
        const int4 dl =
            pre ? zr.dl0 : reinterpret_cast<const int4 *>(a.al.tiles)[min(tb + lu, t1 - 1)];
        asm volatile("" ::"v"(dl.y), "v"(dl.z), "v"(dl.w));
        u32x4_t c0[TB], c1[TB];
#pragma unroll
        for (int u = 0; u < TB; ++u) {
          const int ad = __builtin_amdgcn_readlane(dl.y, lb + u);
          const DT *b0 = Bbase + (((size_t)ad * s.E + e) * b_rows + row) * r;
          c0[u] = load_chunk(b0, kc);
          c1[u] = TWO ? load_chunk(b0 + row_off1 * r, kc) : c0[u];
        }
        static_assert(TB == 8, "one statement reads the whole batch");
        asm volatile("" ::"v"(c0[0]), "v"(c0[1]), "v"(c0[2]), "v"(c0[3]), "v"(c0[4]), "v"(c0[5]),
                     "v"(c0[6]), "v"(c0[7]), "v"(c1[0]), "v"(c1[1]), "v"(c1[2]), "v"(c1[3]),
                     "v"(c1[4]), "v"(c1[5]), "v"(c1[6]), "v"(c1[7]));
#pragma unroll
        for (int u = 0; u < TB; ++u) {
          if (tb + u >= t1) break;
          const int lo = __builtin_amdgcn_readlane(dl.z, lb + u),
                    n = __builtin_amdgcn_readlane(dl.w, lb + u);
          const u32x4_t a0 = kin ? c0[u] : u32x4_t{0, 0, 0, 0};
          const u32x4_t a1 = kin ? c1[u] : u32x4_t{0, 0, 0, 0};
#pragma unroll
          for (int tg = 0; tg < TG; ++tg) {
            // the tile's rows lo .. lo+n-1 miss this 16-row group: it adds nothing
            if (lo >= 16 * (tg + 1) || lo + n <= 16 * tg) continue;
            const int local = tg * 16 + ri;
            const bool in = local >= lo && local < lo + n;
            const u32x4_t zero = u32x4_t{0, 0, 0, 0};
            const u32x4_t h = in ? zh[tg] : zero;
            M::step(acc0[tg], a0, h);
            if (TWO) M::step(acc1[tg], a1, h);
            if constexpr (sizeof(DT) == 2) {
              const u32x4_t l = in ? zl[tg] : zero;
              M::step(acc0[tg], a0, l);
              if (TWO) M::step(acc1[tg], a1, l);
            }
          }
        }
      }
      return;
    }
  }
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
          // z = sum of the shrink's split partials, in split order (row
          // mode: one final z per routed row)
          const float *zp = ROWZ ? a.z + (size_t)prow[tg] * r + kk
                                 : a.z + ((size_t)blk * BM + local) * r + kk;
          const size_t stride = (size_t)s.cap * r;
          const int nsplit = ROWZ ? 1 : a.split;
          if (VEC) {  // r is a multiple of the chunk: whole chunk in or out
            if (kk < r) {
              for (int sp = 0; sp < nsplit; ++sp) {
#pragma unroll
                for (int q = 0; q < EPC; q += 4) {
                  const float4 v4 = *reinterpret_cast<const float4 *>(zp + sp * stride + q);
                  zv[q] += v4.x;
                  zv[q + 1] += v4.y;
                  zv[q + 2] += v4.z;
                  zv[q + 3] += v4.w;
                }
              }
            }
          } else {
            for (int sp = 0; sp < nsplit; ++sp)
#pragma unroll
              for (int q = 0; q < EPC; ++q)
                if (kk + q < r) zv[q] += zp[sp * stride + q];
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

// Token groups (16 rows) of block blk that hold a routed row.  An expert's
// rows fill its blocks from the front and padding sits at the end of its
// last block, so these are the leading groups; the rest are skipped.
template <int TG>
__device__ __forceinline__ int active_groups(const GemmArgs &a, int blk) {
  int n = 0;
#pragma unroll
  for (int tg = 0; tg < TG; ++tg)
    if (a.al.sorted_rows[blk * 16 * TG + tg * 16] < a.s.R) n = tg + 1;
  return n;
}


// gate_up GEMM + expand + SiLU(gate) * up.  Block rows are the expert's
// sorted rows; a wave's 16 h-columns n need weight rows n (gate) and I + n
// (up), so SiLU * up is formed in registers.  h is written for the block's
// real rows (padding rows are skipped by every reader).
// MODE: 0 no LoRA, 1 tile-wise (z per sorted position, split partials),
// 2 row-wise (z per routed row).  S > 0: weights streamed through an S-slot
// LDS ring per wave (contract_dma); SH: with the block's tokens shared by
// the workgroup's kShareWaves waves (contract_shared).
template <typename DT, int TG, int U, bool VEC, bool EVEN_K, int MODE, int S, bool SH = false,
          bool W8 = false>
__global__ __launch_bounds__(256) void k_gate_up(GemmArgs a) {
  constexpr int BM = 16 * TG;
  const Shape &s = a.s;
  const int lane = threadIdx.x & (kWave - 1), wave = threadIdx.x / kWave;
  const int ri = lane & 15, kg = lane >> 4;
  const GemmTile gt = gemm_tile(a, blockIdx.x, (s.I + 16 * a.waves - 1) / (16 * a.waves));
  if (gt.blk < 0) return;
  const int blk = gt.blk;
  const int e = a.al.block_expert[blk];
  const int I = s.I, H = s.H;
  const int n0 = (gt.nt * a.waves + wave) * 16;
  // (SH: a wave past the last column still takes part in the workgroup's
  // token loads and barriers, on clamped rows, and returns after them)
  if (e < 0 || (!SH && n0 >= I)) return;
  const int nrow = min(n0 + ri, I - 1);
  const DT *wg = static_cast<const DT *>(a.W) + ((size_t)e * 2 * I + nrow) * H;
  const DT *wu = wg + (size_t)I * H;
  const DT *xr[TG];
  bool ok[TG];
  int prow[TG];
#pragma unroll
  for (int tg = 0; tg < TG; ++tg) {
    const int p = a.al.sorted_rows[blk * BM + tg * 16 + ri];
    ok[tg] = p < s.R;
    prow[tg] = p;
    // padding rows read the block's first token (same lines as a real lane)
    xr[tg] = static_cast<const DT *>(a.x) +
             (size_t)(ok[tg] ? p / s.k : a.al.sorted_rows[blk * BM] / s.k) * H;
  }
  // LoRA tiles of the block and (batched expand) the lane's z values,
  // fetched ahead of the contraction
  int t0 = 0, t1 = 0;
  ZRows<DT, TG> zr{};
  if (MODE != 0) {
    t0 = a.al.block_tile_start[blk];
    t1 = a.al.block_tile_start[blk + 1];
    if (expand_batched<DT, VEC, MODE == 2>(a))
      load_zrows<DT, TG, MODE == 2>(a, blk, t0, t1, kg, ri, prow, zr);
  }
  f32x4_t ag[TG], au[TG];
#pragma unroll
  for (int tg = 0; tg < TG; ++tg) {
    ag[tg] = f32x4_t{0.f, 0.f, 0.f, 0.f};
    au[tg] = f32x4_t{0.f, 0.f, 0.f, 0.f};
  }
  if constexpr (S > 0) {
    // DMA rows: tile 0 = gate rows n0 .., tile 1 = the matching up rows
    extern __shared__ __align__(16) unsigned char smem[];
    unsigned char *tring = smem;
    int *tok_row = reinterpret_cast<int *>(smem + tok_row_offset(TG, S, W8));
    if constexpr (SH) {
      if (threadIdx.x < BM) {
        const int p = a.al.sorted_rows[blk * BM + threadIdx.x];
        tok_row[threadIdx.x] = (p < s.R ? p : a.al.sorted_rows[blk * BM]) / s.k;
      }
      __syncthreads();
    }
    const int ntg = active_groups<TG>(a, blk);
    if constexpr (W8) {
      const uint8_t *w8[4];  // [tile][instruction]: rows 8 i + lane / 8
#pragma unroll
      for (int i = 0; i < 2; ++i) {
        const uint8_t *g = static_cast<const uint8_t *>(a.W) +
                           ((size_t)e * 2 * I + min(n0 + 8 * i + (lane >> 3), I - 1)) * row_pitch8(H);
        w8[i] = g;
        w8[2 + i] = g + (size_t)I * row_pitch8(H);
      }
      const int c8 = (lane & 7) ^ (lane >> 3);
      const int rot = walk_start8(a, H, gt.nt);
      const float *sc = a.wscale + (size_t)e * 2 * I + min(n0, I - 16);
      const float4 sg = row_scales(sc, kg), su = row_scales(sc + I, kg);
      if constexpr (SH) {
        contract_shared8_groups<TG, 2, S>(w8, 16 * c8, 16 * (c8 & 3), static_cast<const uint16_t *>(a.x),
                                          (size_t)H, tok_row, ntg, H, kg, ri, wave, rot, tring,
                                          tring + S * TG * 4096 + wave * S * 4096, ag, au);
        if (n0 >= I) return;
      } else {
        contract_dma8_groups<TG, 2, S>(w8, 16 * c8, 16 * (c8 & 3),
                                       reinterpret_cast<const uint16_t *const *>(xr), ntg, H, kg, ri,
                                       rot, smem + wave * S * 4096, ag, au);
      }
      // the row scales multiply the base contraction only, before the expand
      scale_rows<TG>(sg, ag);
      scale_rows<TG>(su, au);
    } else {
      const uint16_t *dsrc[4];  // [tile][instruction]
#pragma unroll
      for (int i = 0; i < 2; ++i) {
        const int r = 8 * i + (lane >> 3);
        const uint16_t *g = static_cast<const uint16_t *>(a.W) +
                            ((size_t)e * 2 * I + min(n0 + r, I - 1)) * H + 8 * ((lane & 7) ^ (r & 7));
        dsrc[i] = g;
        dsrc[2 + i] = g + (size_t)I * H;
      }
      if constexpr (SH) {
        contract_shared_groups<TG, 2, S>(dsrc, static_cast<const uint16_t *>(a.x), (size_t)H, tok_row,
                                         ntg, H, kg, ri, wave, walk_start(a, H, gt.nt), tring,
                                         tring + S * TG * 2048 + wave * S * 4096, ag, au);
        if (n0 >= I) return;
      } else {
        contract_dma_groups<TG, 2, S>(dsrc, reinterpret_cast<const uint16_t *const *>(xr), ntg, H, kg,
                                      ri, walk_start(a, H, gt.nt), smem + wave * S * 4096, ag, au);
      }
    }
  } else {
    contract<DT, TG, U, VEC, EVEN_K, true>(wg, wu, xr, active_groups<TG>(a, blk), H, kg, ag, au);
  }
  if (MODE != 0)
    expand<DT, TG, VEC, true, MODE == 2>(a, blk, e, t0, t1, zr, static_cast<const DT *>(a.B),
                                         (size_t)2 * I, nrow, (size_t)I, kg, ri, prow, ag, au);
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

// down GEMM (+ expand when MODE == 1), written per routed row: y[p][m]
// (float).  MODE 2 (row-wise LoRA): the first a.row_wgs workgroups compute
// the down shrink of one routed row each, z_d[p] = h[pos_p] . A_d[a][e]^T,
// alongside the base GEMM (both only need h); the expand then happens in
// the combine.  With a.ksplit > 1 (LDS ring only) the contraction is split
// over workgroups: split q sums its slab range into y[q] (the expand goes to
// split 0), and the combine adds the partials in split order.
template <typename DT, int TG, int U, bool VEC, bool EVEN_K, int MODE, bool R2, int S,
          bool SH = false, bool W8 = false>
__global__ __launch_bounds__(256) void k_down(GemmArgs a) {
  constexpr int BM = 16 * TG;
  const Shape &s = a.s;
  int bid = blockIdx.x;
  if constexpr (MODE == 2) {
    __shared__ float red[256];
    if (bid < a.row_wgs) {
      const int p = bid, t = p / s.k;
      const int ad = a.rs.adapter_ids[t], e = a.topk_ids[p];
      if (ad < 0 || ad >= s.NA || e < 0 || e >= s.E) return;
      const DT *h = static_cast<const DT *>(a.rs.x) + (size_t)a.al.row_pos[p] * s.I;
      const DT *A = static_cast<const DT *>(a.rs.A) + ((size_t)ad * s.E + e) * s.r * s.I;
      row_shrink<DT, VEC>(h, A, s.I, s.r, a.rs.z + (size_t)p * s.r, red);
      return;
    }
    bid -= a.row_wgs;
  }
  const int lane = threadIdx.x & (kWave - 1), wave = threadIdx.x / kWave;
  const int ri = lane & 15, kg = lane >> 4;
  const int I = s.I, H = s.H;
  // column tile and contraction split: the tiles of split q follow those of
  // split q - 1; split q takes slabs [q nsl / ksplit, (q + 1) nsl / ksplit)
  const int cols = (R2 ? 32 : 16) * a.waves;
  const int ntn = (H + cols - 1) / cols;
  const GemmTile gt = gemm_tile(a, bid, ntn * (S > 0 ? a.ksplit : 1));
  if (gt.blk < 0) return;
  const int blk = gt.blk;
  const int e = a.al.block_expert[blk];
  const int ksp = gt.nt / ntn, nt = gt.nt - ksp * ntn;
  int k0 = 0, kn = I;
  if (S > 0 && a.ksplit > 1) {
    const int nsl = I / 64;
    k0 = 64 * (ksp * nsl / a.ksplit);
    kn = 64 * ((ksp + 1) * nsl / a.ksplit) - k0;
  }
  // R2: the wave owns two 16-row tiles (rows m0 .. m0+31), two weight
  // streams against one set of h fragments
  const int m0 = (nt * a.waves + wave) * (R2 ? 32 : 16);
  if (e < 0 || (!SH && m0 >= H)) return;  // (SH: as in k_gate_up)
  const int mrow = min(m0 + ri, H - 1);
  const int mrow1 = R2 ? min(m0 + 16 + ri, H - 1) : mrow;
  const DT *wd = static_cast<const DT *>(a.W) + ((size_t)e * H + mrow) * I;
  const DT *wd1 = static_cast<const DT *>(a.W) + ((size_t)e * H + mrow1) * I;
  const DT *xr[TG];
  bool ok[TG];
  int prow[TG];
#pragma unroll
  for (int tg = 0; tg < TG; ++tg) {
    prow[tg] = a.al.sorted_rows[blk * BM + tg * 16 + ri];
    ok[tg] = prow[tg] < s.R;  // padding rows contribute nothing
    // padding rows read the block's first row (always a routed row): the
    // same lines as a real lane, so they coalesce instead of fetching
    // unwritten rows of h
    xr[tg] = static_cast<const DT *>(a.h) + ((size_t)blk * BM + (ok[tg] ? tg * 16 + ri : 0)) * I + k0;
  }
  int t0 = 0, t1 = 0;
  ZRows<DT, TG> zr{};
  if (MODE == 1) {
    t0 = a.al.block_tile_start[blk];
    t1 = a.al.block_tile_start[blk + 1];
    if (expand_batched<DT, VEC, false>(a)) load_zrows<DT, TG, false>(a, blk, t0, t1, kg, ri, prow, zr);
  }
  f32x4_t acc[TG], acc1[TG];
#pragma unroll
  for (int tg = 0; tg < TG; ++tg) acc[tg] = acc1[tg] = f32x4_t{0.f, 0.f, 0.f, 0.f};
  if constexpr (S > 0) {
    extern __shared__ __align__(16) unsigned char smem[];
    constexpr int NW = R2 ? 2 : 1;
    unsigned char *tring = smem;
    int *tok_row = reinterpret_cast<int *>(smem + tok_row_offset(TG, S, W8));
    if constexpr (SH) {
      if (threadIdx.x < BM)
        tok_row[threadIdx.x] =
            blk * BM + (a.al.sorted_rows[blk * BM + threadIdx.x] < s.R ? (int)threadIdx.x : 0);
      __syncthreads();
    }
    const int ntg = active_groups<TG>(a, blk);
    if constexpr (W8) {
      const uint8_t *w8[2 * NW];  // [tile][instruction]: rows 16 t + 8 i + lane / 8
#pragma unroll
      for (int t = 0; t < NW; ++t)
#pragma unroll
        for (int i = 0; i < 2; ++i)
          w8[2 * t + i] = static_cast<const uint8_t *>(a.W) +
                          ((size_t)e * H + min(m0 + 16 * t + 8 * i + (lane >> 3), H - 1)) *
                              row_pitch8(I) + k0;
      const int c8 = (lane & 7) ^ (lane >> 3);
      const int rot = walk_start8(a, kn, gt.nt);
      const float *sc = a.wscale + (size_t)e * H + min(m0, H - (R2 ? 32 : 16));
      const float4 s0 = row_scales(sc, kg), s1 = R2 ? row_scales(sc + 16, kg) : s0;
      if constexpr (SH) {
        contract_shared8_groups<TG, NW, S>(w8, 16 * c8, 16 * (c8 & 3),
                                           static_cast<const uint16_t *>(a.h) + k0, (size_t)I,
                                           tok_row, ntg, kn, kg, ri, wave, rot, tring,
                                           tring + S * TG * 4096 + wave * S * NW * 2048, acc, acc1);
        if (m0 >= H) return;
      } else {
        contract_dma8_groups<TG, NW, S>(w8, 16 * c8, 16 * (c8 & 3),
                                        reinterpret_cast<const uint16_t *const *>(xr), ntg, kn, kg, ri,
                                        rot, smem + wave * S * NW * 2048, acc, acc1);
      }
      scale_rows<TG>(s0, acc);
      if (R2) scale_rows<TG>(s1, acc1);
    } else {
      const uint16_t *dsrc[2 * NW];  // [tile][instruction]
#pragma unroll
      for (int t = 0; t < NW; ++t)
#pragma unroll
        for (int i = 0; i < 2; ++i) {
          const int r = 16 * t + 8 * i + (lane >> 3);
          dsrc[2 * t + i] = static_cast<const uint16_t *>(a.W) + ((size_t)e * H + min(m0 + r, H - 1)) * I +
                            k0 + 8 * ((lane & 7) ^ (r & 7));
        }
      if constexpr (SH) {
        contract_shared_groups<TG, NW, S>(dsrc, static_cast<const uint16_t *>(a.h) + k0, (size_t)I,
                                          tok_row, ntg, kn, kg, ri, wave, walk_start(a, kn, gt.nt),
                                          tring, tring + S * TG * 2048 + wave * S * NW * 2048, acc,
                                          acc1);
        if (m0 >= H) return;
      } else {
        contract_dma_groups<TG, NW, S>(dsrc, reinterpret_cast<const uint16_t *const *>(xr), ntg, kn,
                                       kg, ri, walk_start(a, kn, gt.nt), smem + wave * S * NW * 2048,
                                       acc, acc1);
      }
    }
  } else {
    contract<DT, TG, U, VEC, EVEN_K, R2>(wd, wd1, xr, active_groups<TG>(a, blk), I, kg, acc, acc1);
  }
  if (MODE == 1 && ksp == 0)
    expand<DT, TG, VEC, R2, false>(a, blk, e, t0, t1, zr, static_cast<const DT *>(a.B), (size_t)H,
                                   mrow, (size_t)(mrow1 - mrow), kg, ri, prow, acc, acc1);
#pragma unroll
  for (int half = 0; half < (R2 ? 2 : 1); ++half) {
    const int mb = m0 + 16 * half + kg * 4;
#pragma unroll
    for (int tg = 0; tg < TG; ++tg) {
      if (!ok[tg]) continue;
      const f32x4_t v4 = half ? acc1[tg] : acc[tg];
      float *dst = a.y + ((size_t)ksp * s.R + prow[tg]) * H + mb;
      if (VEC && mb + 3 < H) {
        *reinterpret_cast<float4 *>(dst) = make_float4(v4[0], v4[1], v4[2], v4[3]);
      } else {
#pragma unroll
        for (int v = 0; v < 4; ++v)
          if (mb + v < H) dst[v] = v4[v];
      }
    }
  }
}

// LoRA shrink z = X A^T for the rows of one LoRA tile; X is x (gate_up,
// rows by token) or h (down, rows by sorted position).  Workgroup (tile,
// split) takes one split of the contraction (split-K across workgroups, so
// the skinny shrink of a decode step spreads over many CUs).  Inside it,
// wave tasks are (16-row group of A, token group, contraction part); when
// there are fewer (row group, token group) pairs than waves the split is cut
// again, those partial sums meet in LDS and are added in part order.  The
// result of split s goes to z_out[s][pos][c]; the expand that consumes z
// adds the splits in split order: no atomics, no scheduling-dependent
// rounding.
template <typename DT, int TG, bool VEC, bool EVEN_K, bool FROM_H, int NWV>
__global__ __launch_bounds__(NWV * kWave) void k_shrink(GemmArgs a) {
  using M = Mma<DT>;
  constexpr int EPC = Elem<DT>::kPerChunk;
  constexpr int KS = M::kK;
  constexpr int BM = 16 * TG;
  // partial sums of the split contraction: [nks][16 * ntg rows][r], at most
  // NWV * 16 * 16 floats (r <= 16 * ncg and nks * ncg * ntg <= NWV)
  __shared__ float part[NWV * 16 * 16];
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
  const int ncg = (r + 15) / 16;
  const int tg_lo = lo / 16, tg_hi = (lo + n - 1) / 16, ntg = tg_hi - tg_lo + 1;
  const int pairs = ncg * ntg;
  const int nks = pairs >= NWV ? 1 : NWV / pairs;
  const int nsteps_all = (K + KS - 1) / KS;
  const int split_beg = (int)((long long)split * nsteps_all / a.split);
  const int split_end = (int)((long long)(split + 1) * nsteps_all / a.split);
  const int nsteps = split_end - split_beg;
  float *dst = a.z_out + (size_t)split * s.cap * r;

  for (int u = wave; u < pairs * nks; u += NWV) {
    const int cg = u % ncg, tg = tg_lo + (u / ncg) % ntg, ks = u / pairs;
    const int s_beg = split_beg + (int)((long long)ks * nsteps / nks);
    const int s_end = split_beg + (int)((long long)(ks + 1) * nsteps / nks);
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
        const bool tail = !EVEN_K && st == nsteps_all - 1;
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
        if (in) dst[pos * r + c] = acc[v];
      } else {
        part[(ks * 16 * ntg + (tg - tg_lo) * 16 + ri) * r + c] = acc[v];
      }
    }
  }
  if (nks == 1) return;
  __syncthreads();
  for (int i = threadIdx.x; i < 16 * ntg * r; i += NWV * kWave) {
    const int row = i / r, c = i % r;
    const int local = tg_lo * 16 + row;
    if (local < lo || local >= lo + n) continue;
    float sum = 0.f;
    for (int ks = 0; ks < nks; ++ks) sum += part[(ks * 16 * ntg + row) * r + c];
    dst[((size_t)blk * BM + local) * r + c] = sum;
  }
}

// out[t] = sum_j w[t][j] * y[t*k + j] in ascending j (float), rounded to
// the layer dtype, where y[p] = y[0][p] + y[1][p] + ... over the down
// GEMM's ksplit contraction partials, in order; rows with an out-of-range
// expert id add nothing.  With
// z_d (row-wise LoRA), each row first gets its down expand added:
// y[p][m] += sum_c z_d[p][c] B_d[a][e][m][c] (the expand is linear, so it
// may follow the base GEMM in a later kernel).
template <typename DT, bool VEC>
__global__ __launch_bounds__(256) void k_combine(Shape s, const int *__restrict__ ids,
                                                 const float *__restrict__ w,
                                                 const float *__restrict__ y, int ksplit, DT *out,
                                                 const float *__restrict__ z_d,
                                                 const DT *__restrict__ B_d,
                                                 const int *__restrict__ aid) {
  const int t = blockIdx.x;
  const int m0 = (blockIdx.y * 256 + threadIdx.x) * 4;
  const int H = s.H;
  if (m0 >= H) return;
  float acc[4] = {0.f, 0.f, 0.f, 0.f};
  const size_t ys = (size_t)s.R * H;  // stride of the contraction partials
  if (VEC) {
    // KB routed rows per batch, their loads issued together (a dropped row
    // reads the token's first row and adds nothing), then added in
    // ascending j: one round trip per batch instead of one per row (the
    // 128-expert step's top-8 combine stage: 7.9 -> 7.5 us)
    constexpr int KB = 8;
    for (int j0 = 0; j0 < s.k; j0 += KB) {
      float4 v[KB];
      float wt[KB];
      bool ok[KB];
#pragma unroll
      for (int u = 0; u < KB; ++u) {
        const int j = min(j0 + u, s.k - 1), p = t * s.k + j;
        const int e = ids[p];
        ok[u] = j0 + u < s.k && e >= 0 && e < s.E;
        const int pp = ok[u] ? p : t * s.k;
        wt[u] = w[pp];
        v[u] = *reinterpret_cast<const float4 *>(y + (size_t)pp * H + m0);
      }
      for (int q = 1; q < ksplit; ++q)
#pragma unroll
        for (int u = 0; u < KB; ++u) {
          const int pp = ok[u] ? t * s.k + j0 + u : t * s.k;
          const float4 u4 = *reinterpret_cast<const float4 *>(y + q * ys + (size_t)pp * H + m0);
          v[u].x += u4.x;
          v[u].y += u4.y;
          v[u].z += u4.z;
          v[u].w += u4.w;
        }
#pragma unroll
      for (int u = 0; u < KB; ++u)
        if (ok[u]) {
          acc[0] += wt[u] * v[u].x;
          acc[1] += wt[u] * v[u].y;
          acc[2] += wt[u] * v[u].z;
          acc[3] += wt[u] * v[u].w;
        }
    }
  }
  for (int j = 0; j < (VEC ? 0 : s.k); ++j) {
    const int p = t * s.k + j;
    const int e = ids[p];
    if (e < 0 || e >= s.E) continue;
    const float wj = w[p];
    const float *yr = y + (size_t)p * H + m0;
    for (int q = 0; q < 4; ++q)
      if (m0 + q < H) {
        float v = yr[q];
        for (int u = 1; u < ksplit; ++u) v += yr[u * ys + q];
        acc[q] += wj * v;
      }
  }
  DT *o = out + (size_t)t * H + m0;
  for (int q = 0; q < 4; ++q)
    if (m0 + q < H) o[q] = Elem<DT>::from_f32(acc[q]);
}

// Row-wise LoRA variant: one thread per output column m, and each routed
// row first gets its down expand, y[p][m] += sum_c z_d[p][c] B_d[a][e][m][c]
// (linear, so it may follow the base GEMM in a later kernel).  A wave's 64
// threads read 64 consecutive rows of B_d, i.e. one contiguous run.  The
// loads of KB routed rows (KB = top-k up to 4) are issued together
// (branch-free: a dropped row reads a valid address and is masked in the
// sum), then the rows are added in ascending j.
constexpr int kRankChunks = 4;  // up-front B chunk loads of the row-wise combine
template <typename DT, bool VEC, int KB>
__global__ __launch_bounds__(64) void k_combine_rows(Shape s, const int *__restrict__ ids,
                                                     const float *__restrict__ w,
                                                     const float *__restrict__ y, int ksplit,
                                                     DT *out,
                                                     const float *__restrict__ z_d,
                                                     const DT *__restrict__ B_d,
                                                     const int *__restrict__ aid) {
  constexpr int EPC = Elem<DT>::kPerChunk;
  const int t = blockIdx.x;
  const int m = blockIdx.y * 64 + threadIdx.x;
  const int H = s.H, r = s.r;
  if (m >= H) return;
  int ad = aid[t];
  const bool lora = ad >= 0 && ad < s.NA;
  if (!lora) ad = 0;
  float acc = 0.f;
  for (int j0 = 0; j0 < s.k; j0 += KB) {
    float v[KB], wt[KB];
    bool ok[KB];
    const DT *b[KB];
    const float *zp[KB];
#pragma unroll
    for (int u = 0; u < KB; ++u) {
      const int j = min(j0 + u, s.k - 1), p = t * s.k + j;
      const int e = ids[p];
      ok[u] = j0 + u < s.k && e >= 0 && e < s.E;
      const int ee = ok[u] ? e : 0, pp = ok[u] ? p : t * s.k;
      v[u] = y[(size_t)pp * H + m];
      for (int q = 1; q < ksplit; ++q) v[u] += y[((size_t)q * s.R + pp) * H + m];
      wt[u] = w[pp];
      b[u] = B_d + (((size_t)ad * s.E + ee) * H + m) * r;
      zp[u] = z_d + (size_t)pp * r;
    }
    if (lora) {
      float sum[KB] = {};
      if (VEC && KB <= 2 && r <= kRankChunks * EPC) {
        // the whole rank in at most kRankChunks chunks: every B chunk of the
        // KB rows is loaded before the first product (a chunk past the rank
        // reloads chunk 0 and is not used), then the same sums in the same
        // order as below (illustrative decode step, top-2: 11.8 -> 10.1 us;
        // with four rows per batch the 16 loads per thread measured slower)
        Chunk<DT> bc[KB][kRankChunks];
#pragma unroll
        for (int u = 0; u < KB; ++u)
#pragma unroll
          for (int c = 0; c < kRankChunks; ++c)
            bc[u][c] = chunk_elems<DT>(load_chunk(b[u], c * EPC < r ? c * EPC : 0));
#pragma unroll
        for (int u = 0; u < KB; ++u)
#pragma unroll
          for (int c = 0; c < kRankChunks; ++c)
            if (c * EPC < r) {
#pragma unroll
              for (int q = 0; q < EPC; ++q)
                sum[u] = __builtin_fmaf(zp[u][c * EPC + q], Elem<DT>::to_f32(bc[u][c].v[q]), sum[u]);
            }
      } else {
        for (int c = 0; c < r; c += EPC) {
          Chunk<DT> bc[KB];
#pragma unroll
          for (int u = 0; u < KB; ++u) bc[u] = chunk_elems<DT>(load_chunk_any<DT, VEC>(b[u], c, r));
#pragma unroll
          for (int u = 0; u < KB; ++u)
#pragma unroll
            for (int q = 0; q < EPC; ++q)
              if (VEC || c + q < r)
                sum[u] = __builtin_fmaf(zp[u][c + q], Elem<DT>::to_f32(bc[u].v[q]), sum[u]);
        }
      }
#pragma unroll
      for (int u = 0; u < KB; ++u) v[u] += sum[u];
    }
#pragma unroll
    for (int u = 0; u < KB; ++u)
      if (ok[u]) acc += wt[u] * v[u];
  }
  out[(size_t)t * H + m] = Elem<DT>::from_f32(acc);
}

// ------------------------------------------------------------- dispatch

// Contraction steps per register set of the double-buffered loop (two sets
// in flight): 4 for 16- and 32-row blocks (6 for the 16-row down, which has
// one weight stream), 2 for 64-row blocks.
template <int TG, bool GATE_UP> constexpr int unroll_for() {
  return TG == 1 && !GATE_UP ? 6 : TG <= 2 ? 4 : 2;
}

template <typename DT, int TG, bool VEC, bool EK, int MODE, int S, bool SH = false, bool W8 = false>
hipError_t launch_gu(const GemmArgs &a, int ntn, hipStream_t st) {
  auto kern = k_gate_up<DT, TG, unroll_for<TG, true>(), VEC, EK, MODE, S, SH, W8>;
  // two 16-row tiles (gate, up) per wave, plus the shared token ring
  const int lds = SH ? shared_lds_bytes(TG, 2, S, W8) : S * 4096 * a.waves;
  if (S > 0) {
    const hipError_t err = hipFuncSetAttribute(reinterpret_cast<const void *>(kern),
                                               hipFuncAttributeMaxDynamicSharedMemorySize, lds);
    if (err != hipSuccess) return err;
  }
  return launch_kernel(kern, dim3(round_up8(ntn * a.s.nblk)), dim3(kWave * a.waves), lds, st, a);
}
template <typename DT, int TG, bool VEC, bool EK, int MODE>
hipError_t go_gate_up(const GemmArgs &a, hipStream_t st) {
  const int cols = 16 * a.waves;
  const int ntn = (a.s.I + cols - 1) / cols;
  if constexpr (sizeof(DT) == 2 && VEC && EK) {
    if (a.wscale) {  // E4M3 weights: through the LDS ring only, 3 or 4 slots
      if (a.s.H % 64 != 0 || a.s.I % 16 != 0) return hipErrorInvalidValue;
      const bool sh = a.tok_share && a.waves == kShareWaves;
      if (a.slots == 4)
        return sh ? launch_gu<DT, TG, VEC, EK, MODE, 4, true, true>(a, ntn, st)
                  : launch_gu<DT, TG, VEC, EK, MODE, 4, false, true>(a, ntn, st);
      return sh ? launch_gu<DT, TG, VEC, EK, MODE, 3, true, true>(a, ntn, st)
                : launch_gu<DT, TG, VEC, EK, MODE, 3, false, true>(a, ntn, st);
    }
    if (a.s.H % 64 == 0) {
      if (a.slots == 2)
        return a.tok_share && a.waves == kShareWaves
                   ? launch_gu<DT, TG, VEC, EK, MODE, 2, true>(a, ntn, st)
                   : launch_gu<DT, TG, VEC, EK, MODE, 2>(a, ntn, st);
      if (a.slots == 3)
        return a.tok_share && a.waves == kShareWaves
                   ? launch_gu<DT, TG, VEC, EK, MODE, 3, true>(a, ntn, st)
                   : launch_gu<DT, TG, VEC, EK, MODE, 3>(a, ntn, st);
      if (a.slots == 4)
        return a.tok_share && a.waves == kShareWaves
                   ? launch_gu<DT, TG, VEC, EK, MODE, 4, true>(a, ntn, st)
                   : launch_gu<DT, TG, VEC, EK, MODE, 4>(a, ntn, st);
    }
  }
  if (a.wscale) return hipErrorInvalidValue;
  return launch_gu<DT, TG, VEC, EK, MODE, 0>(a, ntn, st);
}
template <typename DT, int TG, bool VEC, bool EK, int MODE, bool R2, int S, bool SH = false,
          bool W8 = false>
hipError_t launch_d(const GemmArgs &a, int ntn, hipStream_t st) {
  auto kern = k_down<DT, TG, unroll_for<TG, R2>(), VEC, EK, MODE, R2, S, SH, W8>;
  const int extra = MODE == 2 ? a.row_wgs : 0;
  const int lds = SH ? shared_lds_bytes(TG, R2 ? 2 : 1, S, W8) : S * (R2 ? 4096 : 2048) * a.waves;
  if (S > 0) {
    const hipError_t err = hipFuncSetAttribute(reinterpret_cast<const void *>(kern),
                                               hipFuncAttributeMaxDynamicSharedMemorySize, lds);
    if (err != hipSuccess) return err;
  }
  const int ks = S > 0 ? a.ksplit : 1;
  return launch_kernel(kern, dim3(extra + round_up8(ntn * ks * a.s.nblk)), dim3(kWave * a.waves), lds,
                       st, a);
}
template <typename DT, int TG, bool VEC, bool EK, int MODE, bool R2>
hipError_t go_down_r(const GemmArgs &a, int ntn, hipStream_t st) {
  if constexpr (sizeof(DT) == 2 && VEC && EK) {
    if (a.wscale) {  // E4M3 weights: through the LDS ring only, 3 or 4 slots, no split
      if (a.s.I % 64 != 0 || a.s.H % 16 != 0 || a.ksplit != 1) return hipErrorInvalidValue;
      const bool sh = a.tok_share && a.waves == kShareWaves;
      if (a.slots == 4)
        return sh ? launch_d<DT, TG, VEC, EK, MODE, R2, 4, true, true>(a, ntn, st)
                  : launch_d<DT, TG, VEC, EK, MODE, R2, 4, false, true>(a, ntn, st);
      return sh ? launch_d<DT, TG, VEC, EK, MODE, R2, 3, true, true>(a, ntn, st)
                : launch_d<DT, TG, VEC, EK, MODE, R2, 3, false, true>(a, ntn, st);
    }
    if (a.s.I % 64 == 0) {
      if (a.slots == 2)
        return a.tok_share && a.waves == kShareWaves
                   ? launch_d<DT, TG, VEC, EK, MODE, R2, 2, true>(a, ntn, st)
                   : launch_d<DT, TG, VEC, EK, MODE, R2, 2>(a, ntn, st);
      if (a.slots == 3)
        return a.tok_share && a.waves == kShareWaves
                   ? launch_d<DT, TG, VEC, EK, MODE, R2, 3, true>(a, ntn, st)
                   : launch_d<DT, TG, VEC, EK, MODE, R2, 3>(a, ntn, st);
      if (a.slots == 4)
        return a.tok_share && a.waves == kShareWaves
                   ? launch_d<DT, TG, VEC, EK, MODE, R2, 4, true>(a, ntn, st)
                   : launch_d<DT, TG, VEC, EK, MODE, R2, 4>(a, ntn, st);
    }
  }
  if (a.wscale) return hipErrorInvalidValue;
  return launch_d<DT, TG, VEC, EK, MODE, R2, 0>(a, ntn, st);
}
template <typename DT, int TG, bool VEC, bool EK, int MODE>
hipError_t go_down(const GemmArgs &a, hipStream_t st) {
  const bool r2 = a.down_rows == 32;
  const int cols = (r2 ? 32 : 16) * a.waves;
  const int ntn = (a.s.H + cols - 1) / cols;
  return r2 ? go_down_r<DT, TG, VEC, EK, MODE, true>(a, ntn, st)
            : go_down_r<DT, TG, VEC, EK, MODE, false>(a, ntn, st);
}
template <typename DT, int TG, bool VEC, bool EK, bool FROM_H>
hipError_t go_shrink(const GemmArgs &a, hipStream_t st) {
  if (a.shrink_waves == 4)
    return launch_kernel(k_shrink<DT, TG, VEC, EK, FROM_H, 4>, dim3(a.s.max_tiles, a.split),
                         dim3(4 * kWave), 0, st, a);
  if (a.shrink_waves == 8)
    return launch_kernel(k_shrink<DT, TG, VEC, EK, FROM_H, 8>, dim3(a.s.max_tiles, a.split),
                         dim3(8 * kWave), 0, st, a);
  return launch_kernel(k_shrink<DT, TG, VEC, EK, FROM_H, kShrinkWaves>,
                       dim3(a.s.max_tiles, a.split), dim3(kShrinkWaves * kWave), 0, st, a);
}

// (vec, even_k) in {(1,1), (1,0), (0,0)}: unaligned rows always mask.
#define MOELORA_VEK(GO, DT, TG, V, M)                                                \
  ((V).vec ? ((V).even_k ? GO<DT, TG, true, true, M>(a, st) : GO<DT, TG, true, false, M>(a, st)) \
           : GO<DT, TG, false, false, M>(a, st))

// LoRA mode: 0 none, 1 tile-wise, 2 row-wise.
#define MOELORA_MODES(GO, DT, TG, V)                                                 \
  (mode == 0 ? MOELORA_VEK(GO, DT, TG, V, 0)                                         \
   : mode == 1 ? MOELORA_VEK(GO, DT, TG, V, 1) : MOELORA_VEK(GO, DT, TG, V, 2))
#define MOELORA_GEMM(GO, V)                                                          \
  do {                                                                               \
    const int mode = !(V).lora ? 0 : (V).rowz ? 2 : 1;                                \
    if ((V).tg == 1)                                                                 \
      return (V).bf16 ? MOELORA_MODES(GO, uint16_t, 1, V) : MOELORA_MODES(GO, float, 1, V); \
    if ((V).tg == 2)                                                                 \
      return (V).bf16 ? MOELORA_MODES(GO, uint16_t, 2, V) : MOELORA_MODES(GO, float, 2, V); \
    if ((V).tg == 4)                                                                 \
      return (V).bf16 ? MOELORA_MODES(GO, uint16_t, 4, V) : MOELORA_MODES(GO, float, 4, V); \
    return hipErrorInvalidValue;                                                     \
  } while (0)

#define MOELORA_SHRINK(V, FH)                                                        \
  do {                                                                               \
    if ((V).tg == 1)                                                                 \
      return (V).bf16 ? MOELORA_VEK(go_shrink, uint16_t, 1, V, FH)                   \
                      : MOELORA_VEK(go_shrink, float, 1, V, FH);                     \
    if ((V).tg == 2)                                                                 \
      return (V).bf16 ? MOELORA_VEK(go_shrink, uint16_t, 2, V, FH)                   \
                      : MOELORA_VEK(go_shrink, float, 2, V, FH);                     \
    if ((V).tg == 4)                                                                 \
      return (V).bf16 ? MOELORA_VEK(go_shrink, uint16_t, 4, V, FH)                   \
                      : MOELORA_VEK(go_shrink, float, 4, V, FH);                     \
    if ((V).tg == 8 && (V).bf16) return MOELORA_VEK(go_shrink, uint16_t, 8, V, FH);  \
    return hipErrorInvalidValue;                                                     \
  } while (0)

}  // namespace

hipError_t launch_gate_up(const GemmArgs &a, const GemmVariant &v, hipStream_t st) {
  if (a.s.nblk == 0) return hipSuccess;
  if (a.waves < 1 || a.waves > 4) return hipErrorInvalidValue;
  MOELORA_GEMM(go_gate_up, v);
}

hipError_t launch_down(const GemmArgs &a, const GemmVariant &v, hipStream_t st) {
  if (a.s.nblk == 0) return hipSuccess;
  if (a.waves < 1 || a.waves > 4) return hipErrorInvalidValue;
  MOELORA_GEMM(go_down, v);
}

hipError_t launch_shrink(const GemmArgs &a, const GemmVariant &v, bool from_h, hipStream_t st) {
  if (a.s.max_tiles == 0) return hipSuccess;
  if (a.split < 1) return hipErrorInvalidValue;
  if (from_h) MOELORA_SHRINK(v, true);
  MOELORA_SHRINK(v, false);
}

hipError_t launch_combine(const Shape &s, const int *ids, const float *w, const float *y, int ksplit,
                          void *out, bool bf16, const float *z_d, const void *B_d,
                          const int *adapter_ids, bool vec, hipStream_t st) {
  if (s.T == 0) return hipSuccess;
  if (z_d) {
    const dim3 grid(s.T, (s.H + 63) / 64);
#define MOELORA_COMB(DT, V, KB)                                                                  \
  return launch_kernel(k_combine_rows<DT, V, KB>, grid, dim3(64), 0, st, s, ids, w, y, ksplit, \
                       static_cast<DT *>(out), z_d, static_cast<const DT *>(B_d), adapter_ids)
#define MOELORA_COMB_K(DT, V)                                                                  \
  do {                                                                                         \
    if (s.k == 1) MOELORA_COMB(DT, V, 1);                                                      \
    if (s.k == 2) MOELORA_COMB(DT, V, 2);                                                      \
    MOELORA_COMB(DT, V, 4);                                                                    \
  } while (0)
    if (bf16) {
      if (vec) MOELORA_COMB_K(uint16_t, true);
      MOELORA_COMB_K(uint16_t, false);
    }
    if (vec) MOELORA_COMB_K(float, true);
    MOELORA_COMB_K(float, false);
#undef MOELORA_COMB_K
#undef MOELORA_COMB
  }
  const dim3 grid(s.T, (s.H + 1023) / 1024);
#define MOELORA_COMB(DT, V)                                                                      \
  return launch_kernel(k_combine<DT, V>, grid, dim3(256), 0, st, s, ids, w, y, ksplit,          \
                       static_cast<DT *>(out), static_cast<const float *>(nullptr),             \
                       static_cast<const DT *>(nullptr), static_cast<const int *>(nullptr))
  const bool v4 = s.H % 4 == 0;
  if (bf16) {
    if (v4) MOELORA_COMB(uint16_t, true);
    MOELORA_COMB(uint16_t, false);
  }
  if (v4) MOELORA_COMB(float, true);
  MOELORA_COMB(float, false);
#undef MOELORA_COMB
}

}  // namespace moelora
