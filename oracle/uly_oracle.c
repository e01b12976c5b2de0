/*
 * CPU oracle for the Ulysses sequence-parallel exchange and its fused
 * Q/K RMSNorm + RoPE producer.
 *
 * TEST INFRASTRUCTURE ONLY.  Nothing in the library path may call this
 * file: only the tests, the package smoke check and the CPU-baseline leg of
 * the benchmark load it.  It shares no code, header, table or helper with
 * the HIP library; the two meet only through the seeded inputs.
 *
 * Every routine is a plain nested loop over the definition it cites, with
 * no blocking, fusion or reordering.  Floating point is computed in double.
 *
 * Sources (web pages; cited by title and section):
 *  [CA]  TeleFuser documentation, "Communication Architecture":
 *        "Sequence Parallel Communication / Ulysses" (the two relayouts and
 *        their divisibility rules), "Shared Collective Primitives /
 *        Equal-shape gather" (rank-major stacked gather, pad-then-trim of
 *        unequal heights), "Spatial VAE Communication" (height shards,
 *        halos, zero-filled missing halos at the image edge), and the
 *        ownership table row for parallel_shard.py (sequence padding,
 *        slicing, gathering and restoration).
 *  [UC]  flashinfer UlyssesCommunicator(backend="pcie") PR, "What"
 *        (Transforms: exchange_chunks over a destination-major payload).
 *  [QN]  flashinfer PR #6332 (QkvNormRopeExchangeOverlap), "Description"
 *        (each rank receives its head band of all tokens) and
 *        "Assumptions" (fp32 RMSNorm, eps 1e-6, one [head_dim] weight per
 *        Q and per K, interleaved pairwise RoPE from a per-token cos/sin
 *        table, order: QK-norm then RoPE).
 */
#include <math.h>
#include <stdint.h>
#include <string.h>

/* ------------------------------------------------------------------------
 * Relayout [CA "Ulysses"]: the forward exchange scatters heads and gathers
 * the sequence,
 *     [B, S_local, H, D] on each of P ranks  ->  [B, S_local*P, H/P, D];
 * rank q receives the contiguous head band [q*Hl, (q+1)*Hl) of every
 * token ([QN "Description": "its head band of all tokens"]), and the global
 * token index of rank r's local token s is r*S_local + s.
 *
 * Layouts (all contiguous, rank-major, element size `es` bytes, copied as
 * opaque bytes):
 *     x[P][B][S_l][H][D]        sequence-sharded
 *     y[P][B][P*S_l][H/P][D]    head-sharded
 *
 *     y[q][b][r*S_l + s][j][d] = x[r][b][s][q*Hl + j][d]
 * ---------------------------------------------------------------------- */
int oracle_scatter(const void *x_, void *y_, size_t es, int64_t P, int64_t B,
                   int64_t S_l, int64_t H, int64_t D)
{
    const unsigned char *x = (const unsigned char *)x_;
    unsigned char *y = (unsigned char *)y_;
    if (P <= 0 || H % P != 0)
        return -1; /* [CA "Ulysses"]: heads must divide by the world size */
    int64_t Hl = H / P, S = P * S_l;
    for (int64_t q = 0; q < P; ++q)
        for (int64_t b = 0; b < B; ++b)
            for (int64_t r = 0; r < P; ++r)
                for (int64_t s = 0; s < S_l; ++s)
                    for (int64_t j = 0; j < Hl; ++j)
                        for (int64_t d = 0; d < D; ++d) {
                            int64_t src = ((((r * B + b) * S_l + s) * H) + (q * Hl + j)) * D + d;
                            int64_t dst = ((((q * B + b) * S + (r * S_l + s)) * Hl) + j) * D + d;
                            memcpy(y + dst * es, x + src * es, es);
                        }
    return 0;
}

/* The inverse [CA "Ulysses": the output all-to-all gathers heads and
 * scatters the sequence back], with the same layout names:
 *     o[P][B][S][Hl][D] head-sharded  ->  z[P][B][S/P][H][D]
 *     z[r][b][s][q*Hl + j][d] = o[q][b][r*S_l + s][j][d]
 * The gathered sequence S must divide by P. */
int oracle_gather(const void *o_, void *z_, size_t es, int64_t P, int64_t B,
                  int64_t S, int64_t Hl, int64_t D)
{
    const unsigned char *o = (const unsigned char *)o_;
    unsigned char *z = (unsigned char *)z_;
    if (P <= 0 || S % P != 0)
        return -1; /* [CA "Ulysses"]: gathered sequence divisible by P */
    int64_t S_l = S / P, H = Hl * P;
    for (int64_t r = 0; r < P; ++r)
        for (int64_t b = 0; b < B; ++b)
            for (int64_t s = 0; s < S_l; ++s)
                for (int64_t q = 0; q < P; ++q)
                    for (int64_t j = 0; j < Hl; ++j)
                        for (int64_t d = 0; d < D; ++d) {
                            int64_t src = ((((q * B + b) * S + (r * S_l + s)) * Hl) + j) * D + d;
                            int64_t dst = ((((r * B + b) * S_l + s) * H) + (q * Hl + j)) * D + d;
                            memcpy(z + dst * es, o + src * es, es);
                        }
    return 0;
}

/* Destination-major chunk exchange [UC "What: Transforms", exchange_chunks]:
 * rank r's payload is already packed destination-major, x[r][q][chunk];
 * rank q receives rank r's chunk for it at y[q][r]:
 *     y[q][r][:] = x[r][q][:]
 * Nothing inside a chunk is interleaved. */
void oracle_exchange_chunks(const void *x_, void *y_, int64_t P, int64_t chunk_bytes)
{
    const unsigned char *x = (const unsigned char *)x_;
    unsigned char *y = (unsigned char *)y_;
    for (int64_t r = 0; r < P; ++r)
        for (int64_t q = 0; q < P; ++q)
            memcpy(y + (q * P + r) * chunk_bytes, x + (r * P + q) * chunk_bytes, (size_t)chunk_bytes);
}

/* ------------------------------------------------------------------------
 * QKV projection [QN "Description": the BF16 QKV projection heads the fused
 * call; "Assumptions", exchange algorithm: every rank holds a token shard
 * and the full QKV weight].  The weight is stored output-major, one row of
 * `K` inputs per output column (the usual linear-layer layout):
 *     y[m][n] = sum_k x[m][k] * w[n][k]
 * x[M][K], w[N][K], y[M][N], all double (the 16-bit operands arrive
 * widened exactly); no bias term, as the pages name none.
 * ---------------------------------------------------------------------- */
void oracle_linear(const double *x, const double *w, double *y, int64_t M, int64_t N, int64_t K)
{
    for (int64_t m = 0; m < M; ++m)
        for (int64_t n = 0; n < N; ++n) {
            double acc = 0.0;
            for (int64_t k = 0; k < K; ++k)
                acc += x[m * K + k] * w[n * K + k];
            y[m * N + n] = acc;
        }
}

/* ------------------------------------------------------------------------
 * Per-head RMSNorm then interleaved RoPE [QN "Assumptions"], one row of D
 * values per (token, head):
 *     ms   = (1/D) * sum_i x_i^2
 *     n_i  = x_i / sqrt(ms + eps) * w_i
 *     y_2j   = n_2j * c_j - n_2j+1 * s_j
 *     y_2j+1 = n_2j * s_j + n_2j+1 * c_j
 * where (c_j, s_j) = (cos_tab[pos][j], sin_tab[pos][j]) is the per-token
 * table row of the row's global position.  x and w arrive already widened
 * (exactly) from their 16-bit storage; the table is the fp32 table the
 * operator is given.  rows x[n_rows][D], y[n_rows][D], pos[n_rows].
 * ---------------------------------------------------------------------- */
int oracle_norm_rope_rows(const double *x, double *y, int64_t n_rows, int64_t D,
                          const double *w, double eps, const float *cos_tab,
                          const float *sin_tab, int64_t table_rows,
                          const int64_t *pos)
{
    if (D <= 0 || D % 2 != 0)
        return -1;
    int64_t half = D / 2;
    for (int64_t row = 0; row < n_rows; ++row) {
        const double *xr = x + row * D;
        double *yr = y + row * D;
        int64_t g = pos[row];
        if (g < 0 || g >= table_rows)
            return -2;
        double ss = 0.0;
        for (int64_t i = 0; i < D; ++i)
            ss += xr[i] * xr[i];
        double inv = 1.0 / sqrt(ss / (double)D + eps);
        for (int64_t j = 0; j < half; ++j) {
            double n0 = xr[2 * j] * inv * w[2 * j];
            double n1 = xr[2 * j + 1] * inv * w[2 * j + 1];
            double c = (double)cos_tab[g * half + j];
            double s = (double)sin_tab[g * half + j];
            yr[2 * j] = n0 * c - n1 * s;
            yr[2 * j + 1] = n0 * s + n1 * c;
        }
    }
    return 0;
}

/* ------------------------------------------------------------------------
 * Rotary tables.  The operator consumes a per-token fp32 cos/sin table
 * [QN "Assumptions"]; the pages do not give the frequencies, so the
 * standard inverse-power schedule theta^(-2k/d) is used, evaluated in
 * double and rounded once to fp32.  Rows at or beyond `real_rows` are
 * padding and hold the identity rotation (cos 1, sin 0).
 *
 * 1-D: angle[g][j] = g * theta^(-2j/D).
 * ---------------------------------------------------------------------- */
void oracle_rope_table_1d(float *cos_tab, float *sin_tab, int64_t rows,
                          int64_t real_rows, int64_t D, double theta)
{
    int64_t half = D / 2;
    for (int64_t g = 0; g < rows; ++g)
        for (int64_t j = 0; j < half; ++j) {
            double c = 1.0, s = 0.0;
            if (g < real_rows) {
                double freq = pow(theta, -2.0 * (double)j / (double)D);
                double a = (double)g * freq;
                c = cos(a);
                s = sin(a);
            }
            cos_tab[g * half + j] = (float)c;
            sin_tab[g * half + j] = (float)s;
        }
}

/* 3-D (video latent grid T x Hh x Ww, row-major token order): token g sits
 * at t = g / (Hh*Ww), h = (g / Ww) % Hh, w = g % Ww.  The D/2 pairs are
 * split into three consecutive bands of n_t, n_h, n_w pairs (head-dim
 * widths 2*n_t, 2*n_h, 2*n_w); band a rotates by its own axis coordinate:
 *     angle = pos_a * theta^(-2k / (2*n_a)),  k = pair index inside band. */
void oracle_rope_table_3d(float *cos_tab, float *sin_tab, int64_t rows,
                          int64_t real_rows, int64_t D, int64_t Hh, int64_t Ww,
                          int64_t n_t, int64_t n_h, int64_t n_w, double theta)
{
    int64_t half = D / 2;
    for (int64_t g = 0; g < rows; ++g) {
        int64_t t = g / (Hh * Ww), h = (g / Ww) % Hh, w = g % Ww;
        for (int64_t j = 0; j < half; ++j) {
            double c = 1.0, s = 0.0;
            if (g < real_rows && j < n_t + n_h + n_w) {
                int64_t pos_a, k, width;
                if (j < n_t) {
                    pos_a = t; k = j; width = 2 * n_t;
                } else if (j < n_t + n_h) {
                    pos_a = h; k = j - n_t; width = 2 * n_h;
                } else {
                    pos_a = w; k = j - n_t - n_h; width = 2 * n_w;
                }
                double a = (double)pos_a * pow(theta, -2.0 * (double)k / (double)width);
                c = cos(a);
                s = sin(a);
            }
            cos_tab[g * half + j] = (float)c;
            sin_tab[g * half + j] = (float)s;
        }
    }
}

/* ------------------------------------------------------------------------
 * Sequence padding and restoration (parallel_shard.py's role in [CA]'s
 * ownership table: padding, slicing, gathering, restoration).  The global
 * sequence [B][S][R] (R = one token's row of elements) is padded with zero
 * rows at its tail to S_pad = P*S_l and sliced into rank-major shards
 *     x[r][b][s][:] = full[b][r*S_l + s][:]  if r*S_l + s < S, else 0,
 * and restored by concatenating the shards along the sequence and keeping
 * [0, S).
 * ---------------------------------------------------------------------- */
void oracle_pad_shard(const void *full_, void *x_, size_t es, int64_t P,
                      int64_t B, int64_t S, int64_t S_l, int64_t R)
{
    const unsigned char *full = (const unsigned char *)full_;
    unsigned char *x = (unsigned char *)x_;
    for (int64_t r = 0; r < P; ++r)
        for (int64_t b = 0; b < B; ++b)
            for (int64_t s = 0; s < S_l; ++s)
                for (int64_t i = 0; i < R; ++i) {
                    int64_t g = r * S_l + s;
                    unsigned char *dst = x + ((((r * B + b) * S_l) + s) * R + i) * es;
                    if (g < S)
                        memcpy(dst, full + (((b * S) + g) * R + i) * es, es);
                    else
                        memset(dst, 0, es);
                }
}

void oracle_unshard_trim(const void *x_, void *full_, size_t es, int64_t P,
                         int64_t B, int64_t S, int64_t S_l, int64_t R)
{
    const unsigned char *x = (const unsigned char *)x_;
    unsigned char *full = (unsigned char *)full_;
    for (int64_t b = 0; b < B; ++b)
        for (int64_t g = 0; g < S; ++g)
            for (int64_t i = 0; i < R; ++i) {
                int64_t r = g / S_l, s = g % S_l;
                memcpy(full + (((b * S) + g) * R + i) * es,
                       x + ((((r * B + b) * S_l) + s) * R + i) * es, es);
            }
}

/* ------------------------------------------------------------------------
 * Height-sharded spatial tensors [CA "Spatial VAE Communication",
 * "Equal-shape gather"].  A latent [N][Hh][W] (N = B*C*T) is split by
 * height into P shards of heights h[r] at offsets o[r].
 *
 * Halo split: shard r holds rows o[r]-halo .. o[r]+h[r]+halo-1 of the full
 * tensor; a row outside [0, Hh) is zero (a missing neighbour's halo).  The
 * shards sit rank-major in one buffer of stride hmax + 2*halo rows; rows
 * past h[r] + 2*halo are zero.
 *     sh[r][n][i][:] = full[n][o[r] - halo + i][:]   (0 if outside)
 * ---------------------------------------------------------------------- */
void oracle_spatial_split_halo(const void *full_, void *sh_, size_t es, int64_t P,
                               int64_t N, int64_t Hh, int64_t W, const int64_t *h,
                               const int64_t *o, int64_t hmax, int64_t halo)
{
    const unsigned char *full = (const unsigned char *)full_;
    unsigned char *sh = (unsigned char *)sh_;
    int64_t rows = hmax + 2 * halo;
    for (int64_t r = 0; r < P; ++r)
        for (int64_t n = 0; n < N; ++n)
            for (int64_t i = 0; i < rows; ++i)
                for (int64_t c = 0; c < W; ++c) {
                    unsigned char *dst = sh + ((((r * N) + n) * rows + i) * W + c) * es;
                    int64_t src_row = o[r] - halo + i;
                    if (i < h[r] + 2 * halo && src_row >= 0 && src_row < Hh)
                        memcpy(dst, full + (((n * Hh) + src_row) * W + c) * es, es);
                    else
                        memset(dst, 0, es);
                }
}

/* Rank-major stacked gather of the ranks' core rows (halos dropped), each
 * padded to the maximum local height with zero rows:
 *     st[r][n][i][:] = sh[r][n][halo + i][:]  for i < h[r], else 0. */
void oracle_spatial_gather_stacked(const void *sh_, void *st_, size_t es, int64_t P,
                                   int64_t N, int64_t W, const int64_t *h,
                                   int64_t hmax, int64_t halo)
{
    const unsigned char *sh = (const unsigned char *)sh_;
    unsigned char *st = (unsigned char *)st_;
    int64_t rows = hmax + 2 * halo;
    for (int64_t r = 0; r < P; ++r)
        for (int64_t n = 0; n < N; ++n)
            for (int64_t i = 0; i < hmax; ++i)
                for (int64_t c = 0; c < W; ++c) {
                    unsigned char *dst = st + ((((r * N) + n) * hmax + i) * W + c) * es;
                    if (i < h[r])
                        memcpy(dst, sh + ((((r * N) + n) * rows + (halo + i)) * W + c) * es, es);
                    else
                        memset(dst, 0, es);
                }
}

/* Trim each rank's block to its height and concatenate along the height in
 * rank order:  full[n][o[r] + i][:] = st[r][n][i][:], i < h[r]. */
void oracle_spatial_trim_concat(const void *st_, void *full_, size_t es, int64_t P,
                                int64_t N, int64_t Hh, int64_t W, const int64_t *h,
                                const int64_t *o, int64_t hmax)
{
    const unsigned char *st = (const unsigned char *)st_;
    unsigned char *full = (unsigned char *)full_;
    (void)Hh;
    for (int64_t r = 0; r < P; ++r)
        for (int64_t n = 0; n < N; ++n)
            for (int64_t i = 0; i < h[r]; ++i)
                for (int64_t c = 0; c < W; ++c)
                    memcpy(full + (((n * Hh) + o[r] + i) * W + c) * es,
                           st + ((((r * N) + n) * hmax + i) * W + c) * es, es);
}
