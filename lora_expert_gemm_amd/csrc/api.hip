// C ABI of the MoE-LoRA layer: plan, workspace layout, forward.
//
// The forward enqueues, on the caller's stream and without any host
// synchronisation or allocation:
//   route (only when logits are given) -> align (metadata + scatter) ->
//   gate_up shrink -> gate_up GEMM + expand + SiLU*up -> down shrink ->
//   down GEMM + expand -> top-k combine.
// Grids are sized from upper bounds known on the host; blocks past the
// device-side counts exit at once, so nothing waits for the device.  The
// LoRA kernels are not launched at all when the call has no adapters (the
// early exit of the AWS ML blog "Efficiently serve dozens of fine-tuned
// models with vLLM on Amazon SageMaker AI and Amazon Bedrock", section
// "Execution optimizations"), and nothing is compiled or specialised on the
// token count (same section: recompiling per context length was the cause
// of a tenfold time-to-first-token regression).
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

#include <algorithm>
#include <atomic>
#include <mutex>
#include <new>
#include <vector>

#include "../../include/moelora.h"
#include "kernels.h"

using namespace moelora;

thread_local bool moelora::tl_resolve_only = false;

// Tuning switches, read from the environment once, by moelora_plan, and
// fixed for the plan's lifetime (a forward never reads the environment).
struct Tuning {
  int tg = 0;              // streaming block size in 16-row groups, 1, 2 or 4 (0: by bucket)
  int ksplit_d = 0;        // contraction splits of the streaming down GEMM, 1..8 (0: by grid)
  bool tok_share = true;   // streaming GEMMs: tokens shared by a 4-wave workgroup in LDS
  bool verbose = false;    // a failed launch prints its name and HIP error to stderr
};

// What selects the kernels a forward launches, besides the call's own
// options (LoRA or not; router or caller ids).
struct Selection {
  int BM, waves_gu, waves_d, down_rows, shrink_waves;
  bool row, small_align;
  bool operator==(const Selection &o) const {
    return BM == o.BM && waves_gu == o.waves_gu && waves_d == o.waves_d &&
           down_rows == o.down_rows && shrink_waves == o.shrink_waves && row == o.row &&
           small_align == o.small_align;
  }
};

struct moelora_plan_s {
  moelora_desc d;
  size_t ws_bytes;
  Tuning tune;
  // every distinct selection over the token counts 1..max_tokens, with the
  // first token count that makes it; the devices whose code for all of them
  // has been resolved (bit per device), and the lock of that resolution
  std::vector<std::pair<Selection, int>> selections;
  std::atomic<uint64_t> resolved{0};
  std::mutex resolve_mu;
  int waves_override_gu = 0, waves_override_d = 0;  // 0: the table's choice
  int down_rows = 0;  // streaming down GEMM: weight rows per wave (0: by bucket)
  int slots = kRingSlots;  // streaming GEMMs: LDS ring slots of the weight stream (0: registers)
  bool slots_forced = false;  // slots set by the caller's environment
  bool rotate = true;      // streaming GEMMs: staggered slab walks for 4 KB-multiple weight rows
  // LDS-tiled GEMMs: item order, -1 expert-major (column tile outer, block
  // inner), else column tiles per group (<= 1: none).  The 6400-token
  // prefill: 1947 -> 1912 us with groups of 3 (gate_up 1111 -> 1070, down
  // 640 -> 622; 2: 1922, 4: 1924, 6: 1981); expert-major then takes the
  // gate_up's L2 hit rate from 67 to 76 % and its fetched bytes from 3.44 to
  // 2.46 GB per launch (down 72 -> 78 %, 1.38 -> 1.06 GB) for 1-2 % of time.
  int group = -1;
  int shrink_waves = 0;    // waves per shrink workgroup (0: by tile count)
  // stage timing
  bool timing = false;
  int max_calls = 0, n_calls = 0;
  std::vector<hipEvent_t> ev;  // (MOELORA_N_STAGES + 1) per call
  std::vector<unsigned> recorded;  // per call: bit i set if boundary i was recorded
};

namespace {

constexpr size_t kAlign = 256;
constexpr int kTgSmall = 1, kTgMid = 2, kTgLarge = 4, kTgTiled = 8;

size_t up(size_t v) { return (v + kAlign - 1) / kAlign * kAlign; }

// Token-count bucket (block of 16 * tg rows): weight-streaming blocks of 16,
// 32 or 64 rows sized to hold an expert's rows in one block, blocks of 128
// rows for the LDS-tiled MFMA kernels once experts average 64 rows or more
// (bf16 with 16-byte aligned rows).
bool tiled_ok(const moelora_desc &d) {
  return d.dtype == MOELORA_BF16 && d.hidden % 8 == 0 && d.inter % 8 == 0 && d.rank % 8 == 0;
}
bool tiled_shrink_ok(const moelora_desc &d) { return d.rank <= 64; }
// The 8-wave tiled GEMM takes the LoRA expand as extra contraction slabs:
// needs 64-wide slabs of the base contraction K and of (z hi | z lo) (2r).
bool fused_lora_ok(const moelora_desc &d, int K) {
  return tiled_shrink_ok(d) && d.rank % 32 == 0 && K % 64 == 0;
}
int choose_tg(const moelora_desc &d, const Tuning &tu, int T) {
  const long long rows = (long long)T * d.top_k;
  const long long ne = std::max<long long>(1, std::min<long long>(d.n_experts, rows));
  // Streaming blocks: 16 rows while experts average at most 4 rows, then 32
  // rows (most experts' rows in one block, so their weights stream once,
  // without the register cost of 64-row blocks).
  // tuning sweeps only: a forced streaming block size (1, 2 or 4 groups of 16)
  if (tu.tg) return tu.tg;
  // One expert (a dense layer) at decode size: the grid is one or two blocks
  // wide, so the 128-row tiled kernel leaves most CUs idle (43 workgroups for
  // a 64-token step of the 4096 x 11008 MLP: 698 us).  Up to 64 rows one
  // 64-row block reads each weight once (that step 122 -> 116 us against
  // two 32-row blocks, 111 us with a 4-slot ring); above, 32-row blocks.
  if (d.n_experts == 1 && rows <= 64) return kTgLarge;
  if (d.n_experts == 1 && rows <= 128) return kTgMid;
  if (tiled_ok(d) && rows >= 64 * ne) return kTgTiled;
  if (rows <= 4 * ne) return kTgSmall;
  if (rows <= 32 * ne) return kTgMid;
  return kTgLarge;
}

// Waves per GEMM workgroup and weight rows per wave (measured with the
// weight stream through the LDS ring and tokens loaded per wave; where the
// tokens are shared through LDS, make_layout moves 32-row blocks to 4-wave
// workgroups).  16-row blocks: 4 waves for both
// projections (gate_up: 4 x (16 gate + 16 up) rows, ~2.5 % ahead of 2 waves;
// down: 4 x 16 rows).  32-row blocks: down waves that own two 16-row tiles
// each (2 waves x 32 rows; two weight streams share each h fragment, 6-17 %
// faster there and slower for 16-row blocks); gate_up workgroups of 4 waves
// when the intermediate size is large (4 % ahead at 11008 columns) and of
// one wave otherwise (8 % ahead at 768 columns, where a block has only 48
// column tiles).
int choose_waves(int tg, bool gate_up, int inter, long long ne) {
  if (tg == kTgSmall) return 4;
  // (with one or two experts the block count is too small for 4-wave
  // gate_up workgroups to spread evenly over the CUs: 143 -> 92 us with
  // one-wave workgroups for the dense 64-token step)
  if (tg == kTgMid) return gate_up ? (inter >= 4096 && ne > 2 ? 4 : 1) : 2;
  return 4;
}
int choose_down_rows(int tg) { return tg == kTgMid ? 32 : 16; }

// Contraction splits of the streaming down GEMM (bf16 weight stream through
// the LDS ring).  When the (block, column tile) grid fills under a quarter
// of the chip's workgroup slots -- a dense layer at decode size has one or
// two blocks, i.e. 128 two-wave workgroups for 1536 slots -- the
// contraction is split until it fills them (at most 8 splits of at least 16
// slabs), each split writing its own partial y, which the combine adds in
// split order.  At a third of the slots (the illustrative decode step) the
// split measured 0-9 % slower, hence the quarter.
constexpr int kComputeUnits = 256;  // MI355X
int choose_ksplit(const moelora_desc &d, const Tuning &tu, const Shape &s, int tg, int waves_d,
                  bool share, int down_rows) {
  if (tg == kTgTiled || d.dtype != MOELORA_BF16 || d.inter % 64 != 0) return 1;
  // tuning sweeps only: a forced split count (1..8; every split keeps a slab)
  if (tu.ksplit_d) return std::max(1, std::min(tu.ksplit_d, d.inter / 64));
  const int nw = down_rows == 32 ? 2 : 1;  // 16-row weight tiles per wave
  const int lds = share && waves_d == kShareWaves ? shared_lds_bytes(tg, nw, kRingSlots)
                                                  : kRingSlots * nw * 2048 * waves_d;
  const long long slots = (long long)kComputeUnits * std::max(1, 160 * 1024 / lds);
  const int cols = 16 * nw * waves_d;
  const long long grid = (long long)((s.H + cols - 1) / cols) *
                         std::max<long long>(std::min(s.E, s.R), (s.R + s.BM - 1) / s.BM);
  if (4 * grid > slots) return 1;
  const long long k = std::min<long long>({slots / std::max<long long>(1, grid), 8, d.inter / 64 / 16});
  return (int)std::max<long long>(1, k);
}

// Workgroups sharing one shrink tile's contraction: a decode step has only
// tens of LoRA tiles, so each is split over several CUs.
int choose_split(int tg, int R) {
  if (tg != kTgSmall) return 1;
  return std::max(1, std::min(8, 512 / std::max(R, 1)));
}

// Waves per shrink workgroup: 16 while the (tile, split) grid fits in two
// such workgroups per CU, so each of a decode step's few tiles spreads over
// a whole CU; 8 beyond (many experts of a few rows each: ~700 live tiles of
// a 2236-workgroup grid, gate_up shrink 24 -> 19 us and down shrink 16 ->
// 12 us; 4 waves measured between the two).
int choose_shrink_waves(const Shape &s, int split) {
  return (long long)s.max_tiles * split > 2 * kComputeUnits ? 8 : kShrinkWaves;
}

struct Layout {
  Shape s;
  int waves_gu, waves_d, down_rows, split, ksplit;
  size_t off_error, off_counts, off_ids, off_w, off_sorted, off_bexp, off_seg, off_lseg,
      off_tiles, off_bts, off_bcnt, off_bbase, off_tperm, off_toff, off_rpos, off_zero, off_zgu,
      off_zd, off_h, off_y, total;
};

// The weight stream of a projection runs through the LDS ring (bf16, the
// contraction a multiple of 64), where 4-wave workgroups can share tokens.
bool ring_ok(const moelora_desc &d, int K) { return d.dtype != MOELORA_F32 && K % 64 == 0; }

Layout make_layout(const moelora_desc &d, const Tuning &tu, int T) {
  const bool share = tu.tok_share;
  Layout L{};
  Shape &s = L.s;
  s.T = T;
  s.H = d.hidden;
  s.I = d.inter;
  s.E = d.n_experts;
  s.k = d.top_k;
  s.NA = d.n_adapters;
  s.r = d.rank;
  s.R = T * d.top_k;
  s.BM = 16 * choose_tg(d, tu, T);
  const long long ne = std::min<long long>(s.E, s.R);
  const long long bound = (long long)s.R + ne * (s.BM - 1);
  s.cap = (int)((bound + s.BM - 1) / s.BM * s.BM);
  s.nblk = s.cap / s.BM;
  s.max_seg = (int)std::min<long long>(s.R, (long long)s.E * s.NA);
  s.max_tiles = s.nblk + s.max_seg;
  const int tg = s.BM / 16;
  const long long ne_used = std::max<long long>(1, std::min<long long>(d.n_experts, s.R));
  L.waves_gu = choose_waves(tg, true, d.inter, ne_used);
  L.waves_d = choose_waves(tg, false, d.inter, ne_used);
  L.down_rows = choose_down_rows(tg);
  // Tokens shared by the waves of a workgroup make 4-wave workgroups pay
  // for 32-row blocks too: gate_up always (many-expert 183 -> 176 us, dense
  // 92 -> 82 us); down with 32-row tiles per wave while that grid holds 1024
  // workgroups (many-expert 121 -> 108 us), else with 16-row tiles, which
  // double the grid (the illustrative step's 384 workgroups: 154 us with two
  // unshared waves, 170 us with 32-row tiles, 142 us with 16-row tiles).
  if (tg == kTgMid && share && ring_ok(d, d.hidden)) L.waves_gu = kShareWaves;
  if (tg == kTgMid && share && ring_ok(d, d.inter)) {
    L.waves_d = kShareWaves;
    if ((long long)((s.H + 127) / 128) * s.nblk < 4 * kComputeUnits) L.down_rows = 16;
  }
  const bool share_d = share && ring_ok(d, d.inter);
  L.ksplit = choose_ksplit(d, tu, s, tg, L.waves_d, share_d, L.down_rows);
  if (L.ksplit > 1 && L.waves_d != 4) {
    // split down GEMMs run with four-wave workgroups (the dense 64-token
    // step: 71 -> 56 us with 8 splits)
    L.waves_d = 4;
    L.ksplit = choose_ksplit(d, tu, s, tg, L.waves_d, share_d, L.down_rows);
  }
  L.split = choose_split(tg, s.R);
  const size_t es = d.dtype == MOELORA_F32 ? 4 : 2;
  const size_t NB = (size_t)s.E * (s.NA + 1);
  size_t o = 0;
  auto take = [&](size_t bytes) {
    size_t at = o;
    o = up(o + bytes);
    return at;
  };
  L.off_error = take(4);
  L.off_counts = take(16);
  L.off_ids = take(4ull * s.R);
  L.off_w = take(4ull * s.R);
  L.off_sorted = take(4ull * s.cap);
  L.off_bexp = take(4ull * s.nblk);
  L.off_seg = take(4ull * (s.E + 1));
  L.off_lseg = take(16ull * s.max_seg);
  L.off_tiles = take(16ull * s.max_tiles);
  L.off_bts = take(4ull * (s.nblk + 1));
  L.off_bcnt = take(4 * NB);
  L.off_bbase = take(4 * NB);
  L.off_tperm = take(4ull * T);
  L.off_toff = take(4ull * (s.NA + 2));
  L.off_rpos = take(4ull * s.R);
  L.off_zero = take(128);
  // z: tile-wise [split][cap][r] partial sums (or, same size with split 1,
  // bf16 [cap][2r] hi | lo rows), or row-wise [R][r] (R <= cap)
  L.off_zgu = take(4ull * L.split * s.cap * s.r);
  L.off_zd = take(4ull * L.split * s.cap * s.r);
  L.off_h = take(es * s.cap * s.I);
  L.off_y = take(4ull * L.ksplit * s.R * s.H);
  L.total = o;
  return L;
}

bool aligned(const void *p, size_t a) { return ((uintptr_t)p % a) == 0; }
// Bytes of an activation / output / LoRA element, and of a base-weight element.
size_t elem_bytes(const moelora_desc &d) { return d.dtype == MOELORA_F32 ? 4 : 2; }
size_t weight_bytes(const moelora_desc &d) {
  return d.dtype == MOELORA_BF16_FP8W ? 1 : elem_bytes(d);
}
// E4M3 base weights: the row scales follow the codes at the next 256-byte
// boundary of the weight buffer.
size_t scale_offset(size_t codes) { return (codes + 255) / 256 * 256; }

moelora_status check_desc(const moelora_desc *d) {
  if (!d) return MOELORA_ERR_INVALID_ARG;
  if (d->flags & ~(uint32_t)(MOELORA_FLAG_DETERMINISTIC | MOELORA_FLAG_DEBUG_CHECK_IDS))
    return MOELORA_ERR_UNSUPPORTED;
  if (d->dtype != MOELORA_F32 && d->dtype != MOELORA_BF16 && d->dtype != MOELORA_BF16_FP8W)
    return MOELORA_ERR_UNSUPPORTED;
  // E4M3 weights stream through the LDS ring only: contractions in 64-wide
  // slabs, 16-byte aligned adapter rows
  if (d->dtype == MOELORA_BF16_FP8W &&
      (d->hidden % 64 != 0 || d->inter % 64 != 0 || d->rank % 8 != 0))
    return MOELORA_ERR_UNSUPPORTED;
  if (d->n_experts < 1 || d->n_experts > 1024) return MOELORA_ERR_UNSUPPORTED;
  if (d->n_adapters < 0 || d->n_adapters > 255) return MOELORA_ERR_UNSUPPORTED;
  if ((long long)d->n_experts * (d->n_adapters + 1) > 8448) return MOELORA_ERR_UNSUPPORTED;
  if (d->top_k < 1 || d->top_k > std::min(d->n_experts, 32)) return MOELORA_ERR_UNSUPPORTED;
  if (d->rank < 0 || d->rank > 256) return MOELORA_ERR_UNSUPPORTED;
  if (d->n_adapters > 0 && d->rank < 1) return MOELORA_ERR_UNSUPPORTED;
  if (d->hidden < 1 || d->hidden > 65536 || d->inter < 1 || d->inter > 65536)
    return MOELORA_ERR_UNSUPPORTED;
  if (d->max_tokens < 0 || (long long)d->max_tokens * d->top_k > (1LL << 24))
    return MOELORA_ERR_UNSUPPORTED;
  return MOELORA_OK;
}

GemmVariant variant(const moelora_desc &d, int tg, int K, bool lora, bool rowz = false) {
  GemmVariant v;
  v.bf16 = d.dtype != MOELORA_F32;
  v.w8 = d.dtype == MOELORA_BF16_FP8W;
  const int epc = v.bf16 ? 8 : 4;
  const int ks = v.bf16 ? 32 : 16;
  v.tg = tg;
  v.vec = d.hidden % epc == 0 && d.inter % epc == 0 && (d.rank == 0 || d.rank % epc == 0);
  v.even_k = v.vec && K % ks == 0;
  v.lora = lora;
  v.rowz = rowz;
  return v;
}

// A one-expert layer whose rows fit one 64-row streaming block.
bool dense_one_block(const moelora_desc &d, const Shape &s, int tg) {
  return d.n_experts == 1 && tg == kTgLarge && s.R <= s.BM;
}

// Tile-mode LoRA on the streaming GEMMs with the large-batch alignment (a
// scatter launch): the gate_up shrink rides along with the scatter, one
// workgroup per LoRA segment, when the layer is bf16 with 16-byte aligned
// rows and H a multiple of 32; otherwise it runs as its own launch.
bool fold_gu_shrink(const moelora_desc &d, const Shape &s, int tg, const GemmVariant &vg, bool row) {
  return !row && tg != kTgTiled && s.R > kSmallRows && vg.bf16 && vg.vec && vg.even_k &&
         d.n_adapters > 0 && d.rank > 0;
}

// Row-wise LoRA (decode-sized batches): the shrinks ride along with the
// routing/alignment launch and the down launch, and the down expand moves
// into the combine.  Needs the one-workgroup alignment and down workgroups
// with at least r (rounded up to a power of two) threads.
bool use_row_mode(const Shape &s, bool lora, int waves_d) {
  if (!lora || s.R > kSmallRows || s.BM > 64) return false;
  int rp = 1;
  while (rp < s.r) rp <<= 1;
  return 64 * waves_d >= rp;  // 64 threads per wave
}

// The kernel selection a forward of layout L makes (given LoRA).
Selection selection_of(const moelora_plan_s *p, const Layout &L) {
  Selection sel;
  sel.BM = L.s.BM;
  sel.waves_gu = p->waves_override_gu ? p->waves_override_gu : L.waves_gu;
  sel.waves_d = p->waves_override_d ? p->waves_override_d : L.waves_d;
  sel.down_rows = p->down_rows ? p->down_rows : L.down_rows;
  sel.shrink_waves = p->shrink_waves ? p->shrink_waves : choose_shrink_waves(L.s, L.split);
  sel.row = use_row_mode(L.s, true, sel.waves_d);
  sel.small_align = L.s.R <= kSmallRows;
  return sel;
}

int k_tail(const moelora_desc &d, int K) {
  const int ks = d.dtype == MOELORA_F32 ? 16 : 32;
  return (ks - K % ks) % ks;
}

// A failed launch: MOELORA_ERR_HIP, and with MOELORA_VERBOSE set in the
// environment when the plan was made, a line on stderr naming the launch and
// the HIP error.
moelora_status hip_failure(bool verbose, hipError_t err, const char *what, int line) {
  if (verbose)
    fprintf(stderr, "moelora_forward: %s (api.hip:%d) failed: %s (%d)\n", what, line,
            hipGetErrorString(err), (int)err);
  return MOELORA_ERR_HIP;
}

}  // namespace

extern "C" {

const char *moelora_status_string(moelora_status st) {
  switch (st) {
    case MOELORA_OK: return "ok";
    case MOELORA_ERR_INVALID_ARG: return "invalid argument";
    case MOELORA_ERR_UNSUPPORTED: return "unsupported shape or dtype";
    case MOELORA_ERR_WORKSPACE: return "workspace too small";
    case MOELORA_ERR_HIP: return "HIP runtime error";
    case MOELORA_ERR_DEVICE: return "device error word set";
    case MOELORA_ERR_TOO_LARGE: return "call needs more than the static scratch buffer holds";
  }
  return "unknown status";
}

moelora_status moelora_plan(const moelora_desc *desc, moelora_plan_t *plan,
                            size_t *workspace_bytes) {
  if (!plan || !workspace_bytes) return MOELORA_ERR_INVALID_ARG;
  *plan = nullptr;
  moelora_status st = check_desc(desc);
  if (st != MOELORA_OK) return st;
  moelora_plan_s *p = new (std::nothrow) moelora_plan_s();
  if (!p) return MOELORA_ERR_INVALID_ARG;
  p->d = *desc;
  // tuning sweeps only (none is needed; the defaults are the measured choices)
  if (const char *v = getenv("MOELORA_TOKSHARE")) p->tune.tok_share = atoi(v) != 0;
  p->tune.verbose = getenv("MOELORA_VERBOSE") != nullptr;
  if (const char *v = getenv("MOELORA_TG")) {
    const int tg = atoi(v);
    if (tg == 1 || tg == 2 || tg == 4) p->tune.tg = tg;
  }
  if (const char *v = getenv("MOELORA_KSPLIT_D")) {
    const int k = atoi(v);
    if (k >= 1 && k <= 8) p->tune.ksplit_d = k;
  }
  // tuning sweeps only: force the waves per GEMM workgroup (1..4)
  if (const char *v = getenv("MOELORA_WAVES_GU")) p->waves_override_gu = std::max(0, std::min(4, atoi(v)));
  if (const char *v = getenv("MOELORA_WAVES_D")) p->waves_override_d = std::max(0, std::min(4, atoi(v)));
  if (const char *v = getenv("MOELORA_DOWN_ROWS")) p->down_rows = atoi(v) == 32 ? 32 : atoi(v) == 16 ? 16 : 0;
  if (const char *v = getenv("MOELORA_SLOTS")) {
    p->slots = ring_slots_supported(atoi(v)) ? atoi(v) : 0;
    p->slots_forced = true;
  }
  if (const char *v = getenv("MOELORA_ROTATE")) p->rotate = atoi(v) != 0;
  if (const char *v = getenv("MOELORA_GROUP")) p->group = std::max(-1, std::min(16, atoi(v)));
  if (const char *v = getenv("MOELORA_SHRINK_WAVES"))
    p->shrink_waves = atoi(v) == 4 || atoi(v) == 8 || atoi(v) == kShrinkWaves ? atoi(v) : 0;
  // The largest layout over every token count up to max_tokens.  Sizes are
  // not monotone in T (the shrink and down-GEMM split counts fall as T
  // grows, and the block size changes between buckets), so every T is
  // visited: make_layout is a few dozen integer operations.  The same scan
  // records which kernel selections the token counts make.
  size_t ws = make_layout(p->d, p->tune, 0).total;
  for (int T = 1; T <= p->d.max_tokens; ++T) {
    const Layout L = make_layout(p->d, p->tune, T);
    ws = std::max(ws, L.total);
    const Selection sel = selection_of(p, L);
    if (std::find_if(p->selections.begin(), p->selections.end(),
                     [&](const std::pair<Selection, int> &e) { return e.first == sel; }) ==
        p->selections.end())
      p->selections.emplace_back(sel, T);
  }
  p->ws_bytes = ws;
  *plan = p;
  *workspace_bytes = ws;
  return MOELORA_OK;
}

void moelora_plan_destroy(moelora_plan_t plan) {
  if (!plan) return;
  for (hipEvent_t e : plan->ev) (void)hipEventDestroy(e);
  delete plan;
}

moelora_status moelora_workspace_layout(moelora_plan_t plan, int32_t n_tokens,
                                        moelora_layout *out) {
  if (!plan || !out || n_tokens < 0 || n_tokens > plan->d.max_tokens)
    return MOELORA_ERR_INVALID_ARG;
  const Layout L = make_layout(plan->d, plan->tune, n_tokens);
  memset(out, 0, sizeof *out);
  out->block_m = L.s.BM;
  out->cap = L.s.cap;
  out->nblk = L.s.nblk;
  out->max_seg = L.s.max_seg;
  out->max_tiles = L.s.max_tiles;
  out->off_topk_ids = L.off_ids;
  out->off_topk_w = L.off_w;
  out->off_sorted_rows = L.off_sorted;
  out->off_block_expert = L.off_bexp;
  out->off_seg_start = L.off_seg;
  out->off_lora_seg = L.off_lseg;
  out->off_tiles = L.off_tiles;
  out->off_block_tile_start = L.off_bts;
  out->off_counts = L.off_counts;
  out->off_error = L.off_error;
  return MOELORA_OK;
}

namespace {
// Whether a streaming projection (contraction K, wv waves) runs with shared tokens.
bool shares(const moelora_plan_s *plan, int tg, int wv, int K) {
  return plan->tune.tok_share && tg != kTgTiled && wv == kShareWaves && plan->slots != 0 &&
         ring_ok(plan->d, K);
}
}  // namespace

moelora_status moelora_plan_info(moelora_plan_t plan, int32_t n_tokens, char *buf,
                                 size_t buf_len) {
  if (!plan || !buf || buf_len == 0 || n_tokens < 0 || n_tokens > plan->d.max_tokens)
    return MOELORA_ERR_INVALID_ARG;
  const moelora_desc &d = plan->d;
  const Layout L = make_layout(d, plan->tune, n_tokens);
  const int tg = L.s.BM / 16;
  const GemmVariant vg = variant(d, tg, d.hidden, true), vd = variant(d, tg, d.inter, true);
  const int wgu = plan->waves_override_gu ? plan->waves_override_gu : L.waves_gu;
  const int wd = plan->waves_override_d ? plan->waves_override_d : L.waves_d;
  const int down_rows = plan->down_rows ? plan->down_rows : L.down_rows;
  const int ksplit = vd.bf16 && vd.vec && vd.even_k && d.inter % 64 == 0 && plan->slots != 0 &&
                             tg != kTgTiled
                         ? L.ksplit
                         : 1;
  snprintf(buf, buf_len,
           "dtype=%s block_m=%d tg=%d vec=%d even_k_gu=%d even_k_d=%d k_tail_gu=%d "
           "k_tail_d=%d waves_gu=%d waves_d=%d down_rows=%d down_ksplit=%d lora_mode=%s "
           "shrink_split=%d shrink_waves=%d shrink_gu=%s tok_share_gu=%d tok_share_d=%d cap=%d "
           "workspace=%zu",
           vg.w8 ? "bf16_fp8w" : vg.bf16 ? "bf16" : "f32", L.s.BM, tg, (int)vg.vec, (int)vg.even_k, (int)vd.even_k,
           k_tail(d, d.hidden), k_tail(d, d.inter), wgu, wd, tg == kTgTiled ? 0 : down_rows,
           ksplit, d.n_adapters == 0 ? "none" : use_row_mode(L.s, true, wd) ? "row" : "tile",
           L.split, plan->shrink_waves ? plan->shrink_waves : choose_shrink_waves(L.s, L.split),
           d.n_adapters == 0 ? "none"
           : use_row_mode(L.s, true, wd) ? "routing"
           : fold_gu_shrink(d, L.s, tg, vg, false) ? "scatter" : "kernel",
           (int)shares(plan, tg, wgu, d.hidden), (int)shares(plan, tg, wd, d.inter), L.s.cap, L.total);
  return MOELORA_OK;
}

}  // extern "C"

namespace {

// The layer call behind both forward entry points: `workspace` is the
// caller's buffer (moelora_forward) or this device's static scratch array
// (moelora_forward_noalloc).
moelora_status resolve_kernels(moelora_plan_t plan);

moelora_status forward_impl(moelora_plan_t plan, int32_t n_tokens, const void *x,
                            const float *router_logits, const int32_t *topk_ids,
                            const float *topk_w, const int32_t *adapter_ids,
                            const void *w_gate_up, const void *w_down, const void *lora_a_gu,
                            const void *lora_b_gu, const void *lora_a_d, const void *lora_b_d,
                            void *out, void *workspace, size_t workspace_bytes,
                            moelora_stream_t stream) {
  if (!plan) return MOELORA_ERR_INVALID_ARG;
  const moelora_desc &d = plan->d;
  if (n_tokens < 0 || n_tokens > d.max_tokens) return MOELORA_ERR_INVALID_ARG;
  if (n_tokens == 0) return MOELORA_OK;
  if (!x || !w_gate_up || !w_down || !out || !workspace) return MOELORA_ERR_INVALID_ARG;
  // exactly one routing source: logits, or caller ids with their weights
  const bool own_route = topk_ids == nullptr;
  if (own_route ? (!router_logits || topk_w) : (!topk_w || router_logits))
    return MOELORA_ERR_INVALID_ARG;
  const int n_lora_ptr = !!lora_a_gu + !!lora_b_gu + !!lora_a_d + !!lora_b_d;
  if (n_lora_ptr != 0 && n_lora_ptr != 4) return MOELORA_ERR_INVALID_ARG;
  const bool lora = n_lora_ptr == 4 && adapter_ids && d.n_adapters > 0 && d.rank > 0;
  const void *ptrs16[] = {x, w_gate_up, w_down, out, lora_a_gu, lora_b_gu, lora_a_d, lora_b_d};
  for (const void *p : ptrs16)
    if (p && !aligned(p, 16)) return MOELORA_ERR_INVALID_ARG;
  if (!aligned(workspace, kAlign)) return MOELORA_ERR_INVALID_ARG;

  const Layout L = make_layout(d, plan->tune, n_tokens);
  if (workspace_bytes < L.total || L.total > plan->ws_bytes) return MOELORA_ERR_WORKSPACE;
  char *ws = static_cast<char *>(workspace);
  hipStream_t st = reinterpret_cast<hipStream_t>(stream);
  const Shape &s = L.s;
  const int tg = s.BM / 16;

  AlignBufs al;
  al.sorted_rows = reinterpret_cast<int *>(ws + L.off_sorted);
  al.block_expert = reinterpret_cast<int *>(ws + L.off_bexp);
  al.seg_start = reinterpret_cast<int *>(ws + L.off_seg);
  al.lora_seg = reinterpret_cast<int *>(ws + L.off_lseg);
  al.tiles = reinterpret_cast<int *>(ws + L.off_tiles);
  al.block_tile_start = reinterpret_cast<int *>(ws + L.off_bts);
  al.counts = reinterpret_cast<int *>(ws + L.off_counts);
  al.error = reinterpret_cast<int *>(ws + L.off_error);
  al.bucket_cnt = reinterpret_cast<int *>(ws + L.off_bcnt);
  al.bucket_base = reinterpret_cast<int *>(ws + L.off_bbase);
  al.tok_perm = reinterpret_cast<int *>(ws + L.off_tperm);
  al.tok_off = reinterpret_cast<int *>(ws + L.off_toff);
  al.row_pos = reinterpret_cast<int *>(ws + L.off_rpos);

  // Stage timing: an event at the start and after every stage that launched
  // work; a stage that launched nothing reads as 0 ms (back-to-back events
  // are not free on the device timeline).
  hipEvent_t *ev = nullptr;
  unsigned *rec = nullptr;
  if (plan->timing && plan->n_calls < plan->max_calls && !tl_resolve_only) {
    rec = &plan->recorded[plan->n_calls];
    ev = &plan->ev[(size_t)plan->n_calls++ * (MOELORA_N_STAGES + 1)];
    *rec = 0;
  }
  int stage = 0;
  auto mark = [&](bool launched = true) -> hipError_t {
    const int b = stage++;
    if (!ev || !launched) return hipSuccess;
    *rec |= 1u << b;
    return hipEventRecord(ev[b], st);
  };
#define MOELORA_TRY(expr)                                                            \
  do {                                                                               \
    const hipError_t moelora_err_ = (expr);                                          \
    if (moelora_err_ != hipSuccess) return hip_failure(plan->tune.verbose, moelora_err_, #expr, __LINE__); \
  } while (0)

  const int waves_gu = plan->waves_override_gu ? plan->waves_override_gu : L.waves_gu;
  const int waves_d = plan->waves_override_d ? plan->waves_override_d : L.waves_d;
  const bool row = use_row_mode(s, lora, waves_d);
  const GemmVariant vg = variant(d, tg, d.hidden, lora, row);
  const GemmVariant vd = variant(d, tg, d.inter, lora, row);
  float *z_gu = reinterpret_cast<float *>(ws + L.off_zgu);
  float *z_d = reinterpret_cast<float *>(ws + L.off_zd);
  void *h = ws + L.off_h;

  // (after every host-side check: a rejected call touches no device)
  if (!tl_resolve_only) {
    const moelora_status rs = resolve_kernels(plan);
    if (rs != MOELORA_OK) return rs;
  }
  (void)hipGetLastError();  // an error left pending by an earlier call is not this call's
  MOELORA_TRY(mark());
  int *ids_ws = reinterpret_cast<int *>(ws + L.off_ids);
  float *w_ws = reinterpret_cast<float *>(ws + L.off_w);
  RowShrinkArgs rs_gu{x, lora_a_gu, z_gu, adapter_ids, d.hidden, vg.vec};
  const bool fold_gu = lora && fold_gu_shrink(d, s, tg, vg, row);
  SegShrinkArgs ss_gu{x, lora_a_gu, z_gu, d.hidden};
  MOELORA_TRY(launch_route_align(s, own_route ? router_logits : nullptr, topk_ids, ids_ws, w_ws,
                                 lora ? adapter_ids : nullptr, al, row ? &rs_gu : nullptr,
                                 fold_gu ? &ss_gu : nullptr, vg.bf16, st));
  const int *ids = own_route ? ids_ws : topk_ids;
  const float *wts = own_route ? w_ws : topk_w;
  MOELORA_TRY(mark());

  GemmArgs g{};
  g.s = s;
  g.split = L.split;
  g.shrink_waves = plan->shrink_waves ? plan->shrink_waves : choose_shrink_waves(s, L.split);
  g.tok_share = plan->tune.tok_share;
  g.down_rows = plan->down_rows ? plan->down_rows : L.down_rows;
  g.slots = plan->slots;
  // contraction splits of the down GEMM: only where its weight stream goes
  // through the LDS ring
  g.ksplit = vd.bf16 && vd.vec && vd.even_k && d.inter % 64 == 0 && plan->slots != 0 &&
                     tg != kTgTiled
                 ? L.ksplit
                 : 1;
  g.zero_row = ws + L.off_zero;
  g.group = plan->group;
  const bool t8 = tg == kTgTiled;
  const int z2_gu = lora && t8 && fused_lora_ok(d, d.hidden);
  const int z2_d = lora && t8 && fused_lora_ok(d, d.inter);
  g.topk_ids = ids;
  g.x = x;
  g.al = al;
  g.h = h;
  g.y = reinterpret_cast<float *>(ws + L.off_y);

  if (lora && !row && !fold_gu) {
    GemmArgs a = g;
    a.A = lora_a_gu;
    a.z_out = z_gu;
    a.z2 = z2_gu;
    MOELORA_TRY(tg == kTgTiled && tiled_shrink_ok(d)
                    ? launch_tiled_shrink(a, false, st)
                    : launch_shrink(a, variant(d, tg, d.hidden, true), false, st));
  }
  MOELORA_TRY(mark(lora && !row));
  {
    GemmArgs a = g;
    a.W = w_gate_up;
    if (vg.w8)
      a.wscale = reinterpret_cast<const float *>(
          static_cast<const char *>(w_gate_up) +
          scale_offset((size_t)d.n_experts * 2 * d.inter * row_pitch8(d.hidden)));
    a.B = lora_b_gu;
    a.z = z_gu;
    a.z2 = z2_gu;
    if (fold_gu) a.split = 1;  // the scatter writes z whole
    a.waves = waves_gu;
    // (staggered walks: not for one expert with several blocks, whose blocks
    // all stream the same rows and meet in L2 when they walk in step: the
    // dense 64-token gate_up in 32-row blocks 82 -> 79 us without)
    a.rotate = plan->rotate && (d.n_experts > 1 || s.R <= s.BM) &&
               (size_t)d.hidden * weight_bytes(d) % 4096 == 0;
    // 16-row blocks' gate_up with shared tokens: a 4-slot ring (the decode
    // step: 143 -> 139 us; 32-row blocks lose a workgroup per CU to it and
    // slow down 6-20 %)
    if (tg == kTgSmall && !plan->slots_forced && shares(plan, tg, waves_gu, d.hidden)) a.slots = 4;
    // one 64-row block of a one-expert layer: a 4-slot ring too (the dense
    // 64-token step's gate_up 65 -> 64 us, down 41 -> 38 us)
    if (dense_one_block(d, s, tg) && !plan->slots_forced && shares(plan, tg, waves_gu, d.hidden))
      a.slots = 4;
    MOELORA_TRY(tg == kTgTiled ? launch_tiled(a, true, vg, st) : launch_gate_up(a, vg, st));
  }
  MOELORA_TRY(mark());
  if (lora && !row) {
    GemmArgs a = g;
    a.A = lora_a_d;
    a.z_out = z_d;
    a.z2 = z2_d;
    MOELORA_TRY(tg == kTgTiled && tiled_shrink_ok(d)
                    ? launch_tiled_shrink(a, true, st)
                    : launch_shrink(a, variant(d, tg, d.inter, true), true, st));
  }
  MOELORA_TRY(mark(lora && !row));
  {
    GemmArgs a = g;
    a.W = w_down;
    if (vd.w8)
      a.wscale = reinterpret_cast<const float *>(
          static_cast<const char *>(w_down) +
          scale_offset((size_t)d.n_experts * d.hidden * row_pitch8(d.inter)));
    a.B = lora_b_d;
    a.z = z_d;
    a.z2 = z2_d;
    a.waves = waves_d;
    a.rotate = plan->rotate && (d.n_experts > 1 || s.R <= s.BM) &&
               (size_t)d.inter * weight_bytes(d) % 4096 == 0;
    // E4M3 weights, 16-row blocks with shared tokens: a 4-slot down ring too
    // (the decode step's down 56 -> 53 us; bf16 unchanged by it, 32-row
    // blocks slower)
    if (vd.w8 && tg == kTgSmall && !plan->slots_forced && shares(plan, tg, waves_d, d.inter))
      a.slots = 4;
    if (dense_one_block(d, s, tg) && !plan->slots_forced && shares(plan, tg, waves_d, d.inter))
      a.slots = 4;
    if (row) {
      a.rs = RowShrinkArgs{h, lora_a_d, z_d, adapter_ids, d.inter, vd.vec};
      a.row_wgs = s.R;
    }
    MOELORA_TRY(tg == kTgTiled ? launch_tiled(a, false, vd, st) : launch_down(a, vd, st));
  }
  MOELORA_TRY(mark());
  MOELORA_TRY(launch_combine(s, ids, wts, g.y, g.ksplit, out, d.dtype != MOELORA_F32,
                             row ? z_d : nullptr,
                             lora_b_d, adapter_ids, vd.vec, st));
  MOELORA_TRY(mark());
#undef MOELORA_TRY
  return MOELORA_OK;
}

// Resolve, on the current device, every kernel a forward of this plan can
// launch at any token count, once per device: the dispatch of forward_impl
// runs for each recorded selection, with and without LoRA, from logits and
// from caller ids, with tl_resolve_only set, so its launch sites look their
// kernels up (loading code objects) and launch nothing.  The pointers are
// never dereferenced.
moelora_status resolve_kernels(moelora_plan_t plan) {
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess) return MOELORA_ERR_HIP;
  const uint64_t bit = dev >= 0 && dev < 64 ? 1ull << dev : 0;
  if (bit && (plan->resolved.load(std::memory_order_acquire) & bit)) return MOELORA_OK;
  std::lock_guard<std::mutex> lock(plan->resolve_mu);
  if (bit && (plan->resolved.load(std::memory_order_acquire) & bit)) return MOELORA_OK;
  void *const f = reinterpret_cast<void *>(uintptr_t{1} << 12);  // aligned, never dereferenced
  const float *ff = static_cast<const float *>(f);
  const int32_t *fi = static_cast<const int32_t *>(f);
  moelora_status st = MOELORA_OK;
  tl_resolve_only = true;
  for (const auto &e : plan->selections) {
    for (int lora = 0; lora < 2 && st == MOELORA_OK; ++lora)
      for (int route = 0; route < 2 && st == MOELORA_OK; ++route) {
        const void *lp = lora ? f : nullptr;
        st = forward_impl(plan, e.second, f, route ? ff : nullptr, route ? nullptr : fi,
                          route ? nullptr : ff, lora ? fi : nullptr, f, f, lp, lp, lp, lp, f, f,
                          plan->ws_bytes, nullptr);
      }
    if (st != MOELORA_OK) break;
  }
  tl_resolve_only = false;
  if (st == MOELORA_OK && bit) plan->resolved.fetch_or(bit, std::memory_order_acq_rel);
  return st;
}

// Allocation-free calls: the workspace lives in a file-scope device array.
// Each GPU the library runs on holds its own copy (from the first call on it
// until the process ends).  In host code `scratch` names a host-side stand-in,
// not device memory, so its device address is looked up once per device
// with hipGetSymbolAddress and only that address is handed to kernels.
constexpr size_t kStaticScratchBytes = (size_t)64 << 20;
__device__ __align__(256) unsigned char scratch[kStaticScratchBytes];

constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
std::atomic<void *> g_scratch_ptr[kMaxDevices];

// The device address of this device's scratch array (looked up on the
// first call on the device, with that device current).
moelora_status static_scratch(hipStream_t st, void **ptr) {
  int cur = -1, dev = -1;
  if (hipGetDevice(&cur) != hipSuccess) return MOELORA_ERR_HIP;
  if (hipStreamGetDevice(st, &dev) != hipSuccess) return MOELORA_ERR_HIP;
  // the address belongs to the current device: the stream must run there
  if (dev != cur) return MOELORA_ERR_INVALID_ARG;
  if (cur < 0 || cur >= kMaxDevices) return MOELORA_ERR_UNSUPPORTED;
  void *p = g_scratch_ptr[cur].load(std::memory_order_acquire);
  if (!p) {
    std::lock_guard<std::mutex> lock(g_scratch_mu);
    p = g_scratch_ptr[cur].load(std::memory_order_relaxed);
    if (!p) {
      if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess || !p) return MOELORA_ERR_HIP;
      g_scratch_ptr[cur].store(p, std::memory_order_release);
    }
  }
  *ptr = p;
  return MOELORA_OK;
}

}  // namespace

extern "C" {

moelora_status moelora_forward(moelora_plan_t plan, int32_t n_tokens, const void *x,
                               const float *router_logits, const int32_t *topk_ids,
                               const float *topk_w, const int32_t *adapter_ids,
                               const void *w_gate_up, const void *w_down, const void *lora_a_gu,
                               const void *lora_b_gu, const void *lora_a_d, const void *lora_b_d,
                               void *out, void *workspace, size_t workspace_bytes,
                               moelora_stream_t stream) {
  return forward_impl(plan, n_tokens, x, router_logits, topk_ids, topk_w, adapter_ids, w_gate_up,
                      w_down, lora_a_gu, lora_b_gu, lora_a_d, lora_b_d, out, workspace,
                      workspace_bytes, stream);
}

moelora_status moelora_forward_noalloc(moelora_plan_t plan, int32_t n_tokens, const void *x,
                                       const float *router_logits, const int32_t *topk_ids,
                                       const float *topk_w, const int32_t *adapter_ids,
                                       const void *w_gate_up, const void *w_down,
                                       const void *lora_a_gu, const void *lora_b_gu,
                                       const void *lora_a_d, const void *lora_b_d, void *out,
                                       moelora_stream_t stream) {
  if (!plan) return MOELORA_ERR_INVALID_ARG;
  if (n_tokens < 0 || n_tokens > plan->d.max_tokens) return MOELORA_ERR_INVALID_ARG;
  if (n_tokens == 0) return MOELORA_OK;
  // the size check comes before any device call
  if (make_layout(plan->d, plan->tune, n_tokens).total > kStaticScratchBytes)
    return MOELORA_ERR_TOO_LARGE;
  void *ws = nullptr;
  const moelora_status st = static_scratch(reinterpret_cast<hipStream_t>(stream), &ws);
  if (st != MOELORA_OK) return st;
  return forward_impl(plan, n_tokens, x, router_logits, topk_ids, topk_w, adapter_ids, w_gate_up,
                      w_down, lora_a_gu, lora_b_gu, lora_a_d, lora_b_d, out, ws,
                      kStaticScratchBytes, stream);
}

moelora_status moelora_read_device_error(moelora_plan_t plan, const void *workspace,
                                         int32_t *error_bits, moelora_stream_t stream) {
  if (!plan || !workspace || !error_bits) return MOELORA_ERR_INVALID_ARG;
  hipStream_t st = reinterpret_cast<hipStream_t>(stream);
  if (hipStreamSynchronize(st) != hipSuccess) return MOELORA_ERR_HIP;
  const Layout L = make_layout(plan->d, plan->tune, 0);
  if (hipMemcpy(error_bits, static_cast<const char *>(workspace) + L.off_error, 4,
                hipMemcpyDeviceToHost) != hipSuccess)
    return MOELORA_ERR_HIP;
  return MOELORA_OK;
}

moelora_status moelora_timing_begin(moelora_plan_t plan, int32_t max_calls) {
  if (!plan || max_calls < 1 || plan->timing) return MOELORA_ERR_INVALID_ARG;
  plan->ev.assign((size_t)max_calls * (MOELORA_N_STAGES + 1), nullptr);
  plan->recorded.assign((size_t)max_calls, 0u);
  for (hipEvent_t &e : plan->ev)
    if (hipEventCreate(&e) != hipSuccess) return MOELORA_ERR_HIP;
  plan->timing = true;
  plan->max_calls = max_calls;
  plan->n_calls = 0;
  return MOELORA_OK;
}

moelora_status moelora_timing_end(moelora_plan_t plan, double *stage_ms, int32_t n_stages,
                                  int32_t *n_calls) {
  if (!plan || !plan->timing || !stage_ms || n_stages < 0 || !n_calls)
    return MOELORA_ERR_INVALID_ARG;
  moelora_status rc = MOELORA_OK;
  for (int i = 0; i < n_stages; ++i) stage_ms[i] = 0.0;
  for (int c = 0; c < plan->n_calls && rc == MOELORA_OK; ++c) {
    hipEvent_t *ev = &plan->ev[(size_t)c * (MOELORA_N_STAGES + 1)];
    const unsigned rec = plan->recorded[c];
    if (hipEventSynchronize(ev[MOELORA_N_STAGES]) != hipSuccess) {
      rc = MOELORA_ERR_HIP;
      break;
    }
    int last = 0;  // the latest recorded boundary (boundary 0 always is)
    for (int i = 0; i < (int)MOELORA_N_STAGES; ++i) {
      if (!(rec >> (i + 1) & 1u)) continue;  // stage i launched nothing
      float ms = 0.f;
      if (hipEventElapsedTime(&ms, ev[last], ev[i + 1]) != hipSuccess) {
        rc = MOELORA_ERR_HIP;
        break;
      }
      if (i < n_stages) stage_ms[i] += ms;
      last = i + 1;
    }
  }
  *n_calls = plan->n_calls;
  for (hipEvent_t e : plan->ev) (void)hipEventDestroy(e);
  plan->ev.clear();
  plan->recorded.clear();
  plan->timing = false;
  plan->max_calls = plan->n_calls = 0;
  return rc;
}

}  // extern "C"
