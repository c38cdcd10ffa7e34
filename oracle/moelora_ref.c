/*
 * CPU oracle for one fused MoE expert-FFN layer with multi-LoRA.
 *
 * TEST INFRASTRUCTURE ONLY.  Only the test suite, the smoke check and the
 * benchmark's CPU-baseline leg load this library.  It shares no code, header,
 * table, constant or helper with the GPU library, and the GPU library never
 * calls it.
 *
 * The method comes from the AWS Machine Learning blog post "Efficiently serve
 * dozens of fine-tuned models with vLLM on Amazon SageMaker AI and Amazon
 * Bedrock" (read in its Spanish copy on 7minutos.es and its Chinese copy on
 * qingyuntop.top), cited below as [AWS] with the post's section names:
 *   - "Implementing multi-LoRA inference for MoE models in vLLM" and its
 *     Figure 1 ("Illustration of how MoE-LoRA models work"): a router sends
 *     each token to its most relevant experts and their outputs are
 *     aggregated; each expert is a gate_up projection that widens the hidden
 *     state, then a down projection back; a LoRA adapter on a projection with
 *     base weight W (h_in x h_out) adds A (h_in x r) and B (r x h_out), so
 *     y = xW + xAB; shrink is z = xA and expand is zB; every expert carries an
 *     adapter on both projections, chosen per request.
 *   - "Kernel optimizations": the LoRA result is added to the base output.
 *
 * The post does not state the router formula, the activation, or how gate and
 * up are laid out.  This oracle takes the plainest readings:
 *   - router: softmax over the E logits, keep the k largest, renormalise;
 *   - gate_up output of width 2I = [gate | up], activation SiLU(gate) * up,
 *     SiLU(v) = v / (1 + exp(-v));
 *   - no LoRA scaling factor (the post writes y = xW + xAB);
 *   - adapter id -1 means "no adapter" (base model only);
 *   - the routing weight multiplies each expert's down output, and the k
 *     weighted outputs are summed.
 *
 * Precision.  Every input is widened exactly to double (bf16 by a 16-bit
 * shift) and all arithmetic is double, each sum taken sequentially in
 * ascending index order.  Nothing here is rounded to bf16.
 *
 * Threads.  ref_forward may compute different tokens on different OpenMP
 * threads (tokens are independent; each token's arithmetic runs on one
 * thread in the order written below), so the result does not depend on the
 * thread count.  ref_set_threads fixes the count (0: the OpenMP default).
 *
 * Low-precision base weights (dtype REF_BF16_FP8W).  x, the LoRA weights and
 * the output are bf16 as above; W_gu and W_d hold one byte per element, an
 * OCP 8-bit floating-point E4M3 code, and every weight row carries a float32
 * scale: the weight is scale[row] times the code's value.  The pages name an
 * FP8 fused-MoE path (the aib.vote news item on SageMaker fused-MoE kernel
 * optimizations, second item) without a quantisation scheme; one scale per
 * output row is the reading taken here.
 *
 * Storage (row-major, contraction dimension contiguous):
 *   x        [T][H]
 *   W_gu     [E][2I][H]     rows 0..I-1 gate, rows I..2I-1 up
 *   W_d      [E][H][I]
 *   A_gu     [NA][E][r][H]  (math A is H x r; this is its transpose)
 *   B_gu     [NA][E][2I][r] (math B is r x 2I; this is its transpose)
 *   A_d      [NA][E][r][I]
 *   B_d      [NA][E][H][r]
 *   ids, w   [T][k]         routed row p = t*k + j
 *   adapter  [T]            -1 = none
 */
#include <math.h>
#ifdef _OPENMP
#include <omp.h>
#endif
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

enum { REF_F32 = 0, REF_BF16 = 1, REF_BF16_FP8W = 2 };

/* Element i of an input array of the given storage type, widened to double. */
static inline double ld(const void *p, size_t i, int dtype)
{
    if (dtype == REF_F32)
        return (double)((const float *)p)[i];
    uint32_t u = (uint32_t)((const uint16_t *)p)[i] << 16;
    float f;
    memcpy(&f, &u, sizeof f);
    return (double)f;
}

static double silu(double v) { return v / (1.0 + exp(-v)); }

/*
 * Value of an OCP 8-bit floating-point E4M3 code: sign bit, 4 exponent bits
 * with bias 7, 3 mantissa bits; exponent field 0 holds the subnormals
 * m/8 * 2^-6; the codes with every exponent and mantissa bit set are NaN;
 * there are no infinities (the largest finite magnitude is 1.75 * 2^8 = 448).
 */
double ref_fp8_e4m3(int code)
{
    int s = (code >> 7) & 1, e = (code >> 3) & 15, m = code & 7;
    double v;
    if (e == 15 && m == 7)
        return NAN;
    if (e == 0)
        v = ldexp((double)m / 8.0, -6);
    else
        v = ldexp(1.0 + (double)m / 8.0, e - 7);
    return s ? -v : v;
}

/* Element i of row `row` (rows of length K) of a base-weight array: the
 * layer dtype, or for REF_BF16_FP8W scale[row] times the value of its code
 * (fp8[c] holds the 256 code values). */
static inline double ldw(const void *W, const float *scale, const double *fp8, size_t row,
                         size_t K, size_t i, int dtype)
{
    if (dtype == REF_BF16_FP8W)
        return (double)scale[row] * fp8[((const uint8_t *)W)[row * K + i]];
    return ld(W, row * K + i, dtype);
}

/*
 * Router: for each token, softmax over its E logits, keep the k experts with
 * the largest logits (ties to the lower expert index; selecting on the logits
 * rather than on rounded probabilities), and renormalise the kept
 * probabilities to sum to one.  ids[t][0] is the largest.
 * [AWS] "Implementing multi-LoRA inference for MoE models in vLLM": a router
 * sends each token to its most relevant experts.
 */
int ref_route(int T, int E, int k, const float *logits, int32_t *ids, double *w)
{
    if (T < 0 || E <= 0 || k <= 0 || k > E)
        return -1;
    char *taken = (char *)malloc((size_t)E);
    double *prob = (double *)malloc(sizeof(double) * (size_t)E);
    if (!taken || !prob) {
        free(taken);
        free(prob);
        return -2;
    }
    for (int t = 0; t < T; ++t) {
        const float *l = logits + (size_t)t * E;
        double mx = l[0];
        for (int e = 1; e < E; ++e)
            if (l[e] > mx)
                mx = l[e];
        double denom = 0.0;
        for (int e = 0; e < E; ++e) {
            prob[e] = exp((double)l[e] - mx);
            denom += prob[e];
        }
        for (int e = 0; e < E; ++e)
            prob[e] /= denom;

        memset(taken, 0, (size_t)E);
        double kept = 0.0;
        for (int j = 0; j < k; ++j) {
            int best = -1;
            for (int e = 0; e < E; ++e)
                if (!taken[e] && (best < 0 || l[e] > l[best]))
                    best = e;
            taken[best] = 1;
            ids[(size_t)t * k + j] = best;
            kept += prob[best];
        }
        for (int j = 0; j < k; ++j)
            w[(size_t)t * k + j] = prob[ids[(size_t)t * k + j]] / kept;
    }
    free(taken);
    free(prob);
    return 0;
}

/* Sizes of the alignment arrays for R routed rows. */
void ref_align_sizes(int R, int E, int NA, int BM, int64_t *cap, int64_t *nblk,
                     int64_t *max_seg, int64_t *max_tiles)
{
    int64_t ne = E < R ? E : R;
    int64_t bound = (int64_t)R + ne * (BM - 1);
    int64_t c = (bound + BM - 1) / BM * BM;
    int64_t ms = (int64_t)E * NA;
    if (ms > R)
        ms = R;
    *cap = c;
    *nblk = c / BM;
    *max_seg = ms;
    *max_tiles = c / BM + ms;
}

/*
 * Alignment: the rows grouped per expert, each expert's group padded to a
 * multiple of the block size BM, and inside a group the rows ordered by
 * adapter (base-only rows last), then by row index.  This is the structure a
 * grouped expert GEMM with one shared block size over all four LoRA ops runs
 * on ([AWS] "Implementing multi-LoRA inference for MoE models in vLLM": one
 * GEMM per expert, and expert routing combined with adapter selection;
 * "Tuning kernel configurations for Amazon SageMaker AI and Amazon Bedrock":
 * the four ops share BLOCK_SIZE_M).
 *
 * Outputs (sizes from ref_align_sizes):
 *   sorted_rows[cap]     expert e's rows at seg_start[e].., sentinel R in
 *                        padding and after num_padded
 *   block_expert[nblk]   expert of each BM-row block, -1 past num_padded
 *   seg_start[E+1]       padded start of each expert, seg_start[E] = num_padded
 *   lora_seg[max_seg][4] (expert, adapter, start, len) of each run of rows
 *                        sharing one expert and one adapter >= 0, in (expert,
 *                        adapter) order; unused entries (-1, -1, 0, 0)
 *   tiles[max_tiles][4]  (block, adapter, lo, n): each lora_seg run cut at
 *                        block boundaries, lo/n relative to the block
 *   block_tile_start[nblk+1]  first tile whose block is >= b
 *   counts[3]            num_padded, n_lora_seg, n_tiles
 * Rows whose expert id lies outside [0, E) are dropped; adapter ids outside
 * [0, NA) count as "no adapter".
 */
int ref_align(int T, int k, int E, int NA, int BM, const int32_t *ids,
              const int32_t *adapter_ids, int32_t *sorted_rows,
              int32_t *block_expert, int32_t *seg_start, int32_t *lora_seg,
              int32_t *tiles, int32_t *block_tile_start, int32_t *counts)
{
    if (T < 0 || k <= 0 || E <= 0 || NA < 0 || BM <= 0)
        return -1;
    int R = T * k;
    int64_t cap, nblk, max_seg, max_tiles;
    ref_align_sizes(R, E, NA, BM, &cap, &nblk, &max_seg, &max_tiles);

    /* the adapter rank of a row: its token's adapter, or NA for none */
#define ARANK(p)                                                             \
    ((adapter_ids && adapter_ids[(p) / k] >= 0 && adapter_ids[(p) / k] < NA) \
         ? adapter_ids[(p) / k]                                              \
         : NA)

    seg_start[0] = 0;
    for (int e = 0; e < E; ++e) {
        int c = 0;
        for (int p = 0; p < R; ++p)
            if (ids[p] == e)
                ++c;
        seg_start[e + 1] = seg_start[e] + (c + BM - 1) / BM * BM;
    }
    int num_padded = seg_start[E];

    for (int64_t i = 0; i < cap; ++i)
        sorted_rows[i] = R;
    for (int64_t i = 0; i < max_seg; ++i) {
        lora_seg[4 * i + 0] = -1;
        lora_seg[4 * i + 1] = -1;
        lora_seg[4 * i + 2] = 0;
        lora_seg[4 * i + 3] = 0;
    }
    int nseg = 0;
    for (int e = 0; e < E; ++e) {
        int n = seg_start[e];
        for (int a = 0; a <= NA; ++a) {
            int start = n;
            for (int p = 0; p < R; ++p)
                if (ids[p] == e && ARANK(p) == a)
                    sorted_rows[n++] = p;
            if (a < NA && n > start) {
                lora_seg[4 * nseg + 0] = e;
                lora_seg[4 * nseg + 1] = a;
                lora_seg[4 * nseg + 2] = start;
                lora_seg[4 * nseg + 3] = n - start;
                ++nseg;
            }
        }
    }
#undef ARANK

    for (int64_t b = 0; b < nblk; ++b) {
        block_expert[b] = -1;
        for (int e = 0; e < E; ++e)
            if (seg_start[e] <= b * BM && b * BM < seg_start[e + 1])
                block_expert[b] = e;
    }

    for (int64_t i = 0; i < max_tiles; ++i) {
        tiles[4 * i + 0] = -1;
        tiles[4 * i + 1] = -1;
        tiles[4 * i + 2] = 0;
        tiles[4 * i + 3] = 0;
    }
    int nt = 0;
    for (int s = 0; s < nseg; ++s) {
        int a = lora_seg[4 * s + 1], start = lora_seg[4 * s + 2];
        int end = start + lora_seg[4 * s + 3];
        for (int b = start / BM; b <= (end - 1) / BM; ++b) {
            int lo = start > b * BM ? start : b * BM;
            int hi = end < (b + 1) * BM ? end : (b + 1) * BM;
            tiles[4 * nt + 0] = b;
            tiles[4 * nt + 1] = a;
            tiles[4 * nt + 2] = lo - b * BM;
            tiles[4 * nt + 3] = hi - lo;
            ++nt;
        }
    }
    for (int64_t b = 0; b <= nblk; ++b) {
        int first = nt;
        for (int i = nt - 1; i >= 0; --i)
            if (tiles[4 * i + 0] >= b)
                first = i;
        block_tile_start[b] = first;
    }
    counts[0] = num_padded;
    counts[1] = nseg;
    counts[2] = nt;
    return 0;
}

/*
 * The layer for the tokens listed in `tokens` (n_sel of them; all T when
 * tokens is NULL).  out_sel[s][m] receives token tokens[s]'s output, in
 * double.  For each routed row of the token (j ascending):
 *     g   = x W_gu[e]^T            + [a >= 0] (x A_gu[a][e]^T) B_gu[a][e]^T
 *     h   = SiLU(g[0:I]) * g[I:2I]
 *     y   = h W_d[e]^T             + [a >= 0] (h A_d[a][e]^T)  B_d[a][e]^T
 *     out += w[t][j] * y
 * [AWS] "Implementing multi-LoRA inference for MoE models in vLLM" (Figure 1;
 * the four LoRA ops gate_up shrink/expand and down shrink/expand per expert,
 * per adapter, per request) and "Kernel optimizations" (the expand result is
 * added into the base output).  Rows with an expert id outside [0, E) add
 * nothing; adapter ids outside [0, NA) mean no adapter.  Null LoRA pointers
 * mean no adapter for any token.
 */
/* One selected token's output row o[H] (see ref_forward); g, h, y, z are
 * scratch rows of 2I, I, H and max(r, 1) doubles. */
static void ref_token(int t, int T, int H, int I, int E, int k, int NA, int r, int dtype,
                      int lora, const void *x, const int32_t *ids, const double *w,
                      const int32_t *adapter_ids, const void *W_gu, const void *W_d,
                      const void *A_gu, const void *B_gu, const void *A_d,
                      const void *B_d, const float *s_gu, const float *s_d,
                      const double *fp8, double *o, double *g, double *h, double *y,
                      double *z)
{
    size_t I2 = 2 * (size_t)I;
    for (int m = 0; m < H; ++m)
        o[m] = 0.0;
    if (t < 0 || t >= T)
        return;
    int a = lora ? adapter_ids[t] : -1;
    if (a < 0 || a >= NA)
        a = -1;
    for (int j = 0; j < k; ++j) {
        int e = ids[(size_t)t * k + j];
        if (e < 0 || e >= E)
            continue;
        /* gate_up: base, then shrink and expand */
        for (size_t n = 0; n < I2; ++n) {
            double acc = 0.0;
            size_t wrow = (size_t)e * I2 + n;
            for (int c = 0; c < H; ++c)
                acc += ld(x, (size_t)t * H + c, dtype) *
                       ldw(W_gu, s_gu, fp8, wrow, (size_t)H, (size_t)c, dtype);
            g[n] = acc;
        }
        if (a >= 0) {
            size_t pair = (size_t)a * E + e;
            for (int c = 0; c < r; ++c) {
                double acc = 0.0;
                size_t arow = (pair * r + c) * H;
                for (int q = 0; q < H; ++q)
                    acc += ld(x, (size_t)t * H + q, dtype) * ld(A_gu, arow + q, dtype);
                z[c] = acc;
            }
            for (size_t n = 0; n < I2; ++n) {
                double acc = 0.0;
                size_t brow = (pair * I2 + n) * r;
                for (int c = 0; c < r; ++c)
                    acc += z[c] * ld(B_gu, brow + c, dtype);
                g[n] += acc;
            }
        }
        /* activation */
        for (int i = 0; i < I; ++i)
            h[i] = silu(g[i]) * g[(size_t)I + i];
        /* down: base, then shrink and expand */
        for (int m = 0; m < H; ++m) {
            double acc = 0.0;
            size_t wrow = (size_t)e * H + m;
            for (int i = 0; i < I; ++i)
                acc += h[i] * ldw(W_d, s_d, fp8, wrow, (size_t)I, (size_t)i, dtype);
            y[m] = acc;
        }
        if (a >= 0) {
            size_t pair = (size_t)a * E + e;
            for (int c = 0; c < r; ++c) {
                double acc = 0.0;
                size_t arow = (pair * r + c) * I;
                for (int i = 0; i < I; ++i)
                    acc += h[i] * ld(A_d, arow + i, dtype);
                z[c] = acc;
            }
            for (int m = 0; m < H; ++m) {
                double acc = 0.0;
                size_t brow = (pair * H + m) * r;
                for (int c = 0; c < r; ++c)
                    acc += z[c] * ld(B_d, brow + c, dtype);
                y[m] += acc;
            }
        }
        /* routing-weighted sum over the k experts */
        double wj = w[(size_t)t * k + j];
        for (int m = 0; m < H; ++m)
            o[m] += wj * y[m];
    }
}

static int ref_threads = 0;

/* Threads of ref_forward (0: the OpenMP default); returns the count a call
 * will use. */
int ref_set_threads(int n)
{
    ref_threads = n > 0 ? n : 0;
#ifdef _OPENMP
    return ref_threads ? ref_threads : omp_get_max_threads();
#else
    return 1;
#endif
}

int ref_forward(int T, int H, int I, int E, int k, int NA, int r, int dtype,
                const void *x, const int32_t *ids, const double *w,
                const int32_t *adapter_ids, const void *W_gu, const void *W_d,
                const void *A_gu, const void *B_gu, const void *A_d,
                const void *B_d, const int32_t *tokens, int n_sel,
                double *out_sel, const float *W_gu_scale, const float *W_d_scale)
{
    if (T < 0 || H <= 0 || I <= 0 || E <= 0 || k <= 0 || NA < 0 || r < 0)
        return -1;
    if (dtype < REF_F32 || dtype > REF_BF16_FP8W ||
        (dtype == REF_BF16_FP8W && (!W_gu_scale || !W_d_scale)))
        return -1;
    double fp8[256];
    for (int c = 0; c < 256; ++c)
        fp8[c] = ref_fp8_e4m3(c);
    int lora = A_gu && B_gu && A_d && B_d && adapter_ids && NA > 0 && r > 0;
    int nsel = tokens ? n_sel : T;
    int fail = 0;
#ifdef _OPENMP
    int nt = ref_threads ? ref_threads : omp_get_max_threads();
#pragma omp parallel num_threads(nt) reduction(| : fail)
#endif
    {
        double *g = (double *)malloc(sizeof(double) * 2 * (size_t)I);
        double *h = (double *)malloc(sizeof(double) * (size_t)I);
        double *y = (double *)malloc(sizeof(double) * (size_t)H);
        double *z = (double *)malloc(sizeof(double) * (size_t)(r > 0 ? r : 1));
        if (!g || !h || !y || !z)
            fail = 1;
#ifdef _OPENMP
#pragma omp for schedule(dynamic, 1)
#endif
        for (int s = 0; s < nsel; ++s) {
            if (fail)
                continue;
            ref_token(tokens ? tokens[s] : s, T, H, I, E, k, NA, r, dtype, lora, x, ids, w,
                      adapter_ids, W_gu, W_d, A_gu, B_gu, A_d, B_d, W_gu_scale, W_d_scale,
                      fp8, out_sel + (size_t)s * H, g, h, y, z);
        }
        free(g);
        free(h);
        free(y);
        free(z);
    }
    return fail ? -2 : 0;
}
