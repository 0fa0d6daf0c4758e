/*
 * Plain fp64 CPU oracle for the absorbed-weight sparse MLA decode step.
 *
 * TEST INFRASTRUCTURE ONLY.  Nothing in the product path may include, link
 * or call this file; only the tests, the smoke check and the benchmark's CPU
 * baseline leg do.  It shares no code, header or constant with the HIP
 * library.
 *
 * Source of every step (DeepSeek-V3.2-Exp pages):
 *   "Query-key similarity" page, formula S_i and the decode-branch code
 *       excerpt: absorption of W_UK into the query, the two score terms
 *       (latent and rotary), the softmax scale, the -inf index mask built by
 *       scattering zeros at the selected positions, the softmax over keys,
 *       the latent mix and the W_UV projection.
 *   "Queries" page, init excerpt: softmax_scale = qk_head_dim^-1/2, the
 *       wkv_b weight of n_heads*(qk_nope_head_dim + v_head_dim) rows by
 *       kv_lora_rank columns.
 *   "Softmax" page, formula for A: normalisation over key positions.
 *   "Apply value weights" page, formula O_i = O~_i W_UV,i.
 *
 * This is the gather formulation: it sums only over the selected set, which
 * equals the dense masked sum because exp(-inf) contributes exactly zero.
 * It is pinned against the dense masked and the non-absorbed formulations,
 * closed forms and a library attention routine by the CPU tests.
 *
 * Every float value is handled in IEEE double.  No blocking, fusion or
 * reordering: each output is the literal sum, accumulated in index order.
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

#define ORACLE_OK 0
#define ORACLE_ERR_INDEX_RANGE 1   /* an index >= L_b, or negative and not -1 */
#define ORACLE_ERR_EMPTY 4         /* a sequence has no selected position      */
#define ORACLE_ERR_ARG 8           /* bad sizes or pointers                    */

/*
 * Decode an OCP FP8 E4M3FN byte (1 sign, 4 exponent bits with bias 7,
 * 3 mantissa bits, no infinities, 0x7F/0xFF are NaN) to double.
 */
double oracle_e4m3_to_double(uint8_t code) {
    int s = (code >> 7) & 1;
    int e = (code >> 3) & 15;
    int m = code & 7;
    double v;
    if (e == 15 && m == 7) return NAN;
    if (e == 0) v = ldexp((double)m / 8.0, -6);            /* subnormal */
    else v = ldexp(1.0 + (double)m / 8.0, e - 7);          /* normal    */
    return s ? -v : v;
}

/* Round a double to the nearest bfloat16 (8 significant bits), ties to even,
 * and return its 16-bit pattern.  Values here are far from overflow. */
uint16_t oracle_double_to_bf16(double x) {
    if (isnan(x)) return 0x7FC0;
    if (x == 0.0) return signbit(x) ? 0x8000 : 0x0000;
    double ax = fabs(x);
    int e;
    frexp(ax, &e);                   /* ax = f * 2^e with f in [0.5, 1) */
    int q = e - 8;                   /* ulp of an 8-bit significand     */
    if (q < -133) q = -133;          /* bf16 subnormal spacing          */
    double r = rint(ldexp(ax, -q));  /* default rounding: ties to even  */
    double y = ldexp(r, q);
    float f = (float)y;              /* exact: y has <= 8 significant bits */
    uint32_t bits;
    memcpy(&bits, &f, 4);
    bits >>= 16;
    if (x < 0) bits |= 0x8000;
    return (uint16_t)bits;
}

/*
 * Dequantise a block-scaled FP8 weight: W[i][j] = bf16_RNE(e4m3(w[i][j]) *
 * scale[i / blk][j / blk]).  The product of an e4m3 value (4 significant
 * bits) and an fp32 scale (24 bits) is exact in double, so the only rounding
 * is the final one to bf16.  Optionally also writes the exact product.
 */
int oracle_dequant_fp8(const uint8_t* w, const float* scales, int64_t rows,
                       int64_t cols, int64_t blk, uint16_t* out_bf16,
                       double* out_exact) {
    if (!w || !scales || rows <= 0 || cols <= 0 || blk <= 0) return ORACLE_ERR_ARG;
    int64_t scols = (cols + blk - 1) / blk;
    for (int64_t i = 0; i < rows; ++i)
        for (int64_t j = 0; j < cols; ++j) {
            double v = oracle_e4m3_to_double(w[i * cols + j]) *
                       (double)scales[(i / blk) * scols + (j / blk)];
            if (out_exact) out_exact[i * cols + j] = v;
            if (out_bf16) out_bf16[i * cols + j] = oracle_double_to_bf16(v);
        }
    return ORACLE_OK;
}

/*
 * The selected set M_b of one sequence: the distinct in-range positions named
 * by its index row (the mask is built by scattering a constant, so a repeat
 * counts once).  -1 is padding and is skipped.  Returns the set size, or -1
 * if an index is out of range.  `mark` is scratch of length L.
 */
static int64_t selected_set(const int64_t* idx, int64_t k, int64_t L,
                            unsigned char* mark, int64_t* set) {
    memset(mark, 0, (size_t)L);
    for (int64_t j = 0; j < k; ++j) {
        int64_t t = idx[j];
        if (t == -1) continue;
        if (t < 0 || t >= L) return -1;
        mark[t] = 1;
    }
    int64_t n = 0;
    for (int64_t t = 0; t < L; ++t)
        if (mark[t]) set[n++] = t;
    return n;
}

/*
 * One absorbed sparse decode step for B sequences.
 *
 *   q_nope [B][H][Dn], q_pe [B][H][Dr]          (contiguous)
 *   kv: latent row of (b, t) at kv + b*kv_sb + t*kv_st, Dc contiguous values
 *   pe: rotary row of (b, t) at pe + b*pe_sb + t*pe_st, Dr contiguous values
 *   wkv_b [H*(Dn+Dv)][Dc]: viewed per head as [H][Dn+Dv][Dc]; the first Dn
 *       rows of a head are W_UK (stored [d][c]), the last Dv rows are W_UV.
 *   seq_lens [B]: cached positions L_b.
 *   indices [B][k_max] or NULL.  NULL selects every position t < L_b.
 *   scale: the softmax scale applied to the summed scores.
 *
 * Outputs (any may be NULL except out):
 *   q_abs  [B][H][Dc]  absorbed query
 *   o_lat  [B][H][Dc]  normalised latent mix O~
 *   out    [B][H][Dv]  head outputs O
 *   lse    [B][H]      natural-log log-sum-exp of the masked scores
 *   attended [B][att_stride]  1 where position t is in M_b, else 0
 *   weights [B][H][k_max]  softmax weight of the position named by each
 *       index slot (0 for padding); a repeated position reports its weight
 *       once per slot it appears in.  Only with indices != NULL.
 *   scores  [B][H][k_max]  scaled score of each slot's position (-inf for
 *       padding).  Only with indices != NULL.
 *
 * Returns a bit set of ORACLE_ERR_* (0 = OK).  An empty selection yields NaN
 * outputs for that sequence, as the softmax of an all -inf row does.
 */
int oracle_decode(int64_t B, int64_t H, int64_t Dn, int64_t Dc, int64_t Dr,
                  int64_t Dv, const double* q_nope, const double* q_pe,
                  const double* kv, int64_t kv_sb, int64_t kv_st,
                  const double* pe, int64_t pe_sb, int64_t pe_st,
                  const double* wkv_b, const int32_t* seq_lens,
                  const int64_t* indices, int64_t k_max, double scale,
                  double* q_abs, double* o_lat, double* out, double* lse,
                  unsigned char* attended, int64_t att_stride,
                  double* weights, double* scores) {
    if (B <= 0 || H <= 0 || Dn <= 0 || Dc <= 0 || Dr < 0 || Dv <= 0 ||
        !q_nope || !kv || !wkv_b || !seq_lens || !out || (Dr > 0 && (!q_pe || !pe)))
        return ORACLE_ERR_ARG;
    if (indices && k_max <= 0) return ORACLE_ERR_ARG;
    int status = ORACLE_OK;
    const int64_t rows_per_head = Dn + Dv;

    for (int64_t b = 0; b < B; ++b) {
        const int64_t L = seq_lens[b];
        if (L < 0) return ORACLE_ERR_ARG;

        /* Step 4 (mask): the selected set of this sequence, shared by every
         * head because the mask is broadcast over the head dimension. */
        int64_t* set = (int64_t*)malloc(sizeof(int64_t) * (size_t)(L > 0 ? L : 1));
        unsigned char* mark = (unsigned char*)malloc((size_t)(L > 0 ? L : 1));
        int64_t n;
        if (indices) {
            n = selected_set(indices + b * k_max, k_max, L, mark, set);
            if (n < 0) { free(set); free(mark); return status | ORACLE_ERR_INDEX_RANGE; }
        } else {
            for (int64_t t = 0; t < L; ++t) set[t] = t;
            n = L;
        }
        if (n == 0) status |= ORACLE_ERR_EMPTY;
        if (attended) {
            memset(attended + b * att_stride, 0, (size_t)att_stride);
            for (int64_t j = 0; j < n; ++j) attended[b * att_stride + set[j]] = 1;
        }

        #pragma omp parallel for schedule(dynamic, 1)
        for (int64_t h = 0; h < H; ++h) {
            const double* w_uk = wkv_b + (h * rows_per_head) * Dc;        /* [Dn][Dc] */
            const double* w_uv = wkv_b + (h * rows_per_head + Dn) * Dc;   /* [Dv][Dc] */
            const double* qn = q_nope + (b * H + h) * Dn;
            const double* qr = Dr > 0 ? q_pe + (b * H + h) * Dr : NULL;
            double* qa = (double*)malloc(sizeof(double) * (size_t)Dc);
            double* s = (double*)malloc(sizeof(double) * (size_t)(n > 0 ? n : 1));
            double* mix = (double*)malloc(sizeof(double) * (size_t)Dc);

            /* Step 2 (absorb): q~[c] = sum_d q_nope[d] * W_UK[d][c]. */
            for (int64_t c = 0; c < Dc; ++c) {
                double acc = 0.0;
                for (int64_t d = 0; d < Dn; ++d) acc += qn[d] * w_uk[d * Dc + c];
                qa[c] = acc;
            }

            /* Step 3 (scores): s_t = scale * (q~ . c_t + q_pe . k_pe_t). */
            for (int64_t j = 0; j < n; ++j) {
                const double* crow = kv + b * kv_sb + set[j] * kv_st;
                double lat = 0.0, rot = 0.0;
                for (int64_t c = 0; c < Dc; ++c) lat += qa[c] * crow[c];
                if (Dr > 0) {
                    const double* prow = pe + b * pe_sb + set[j] * pe_st;
                    for (int64_t r = 0; r < Dr; ++r) rot += qr[r] * prow[r];
                }
                s[j] = (lat + rot) * scale;
            }

            /* Step 5 (softmax over the keys): A_t = exp(s_t - m) / sum_u exp(s_u - m). */
            double m = -INFINITY;
            for (int64_t j = 0; j < n; ++j) if (s[j] > m) m = s[j];
            double denom = 0.0;
            for (int64_t j = 0; j < n; ++j) denom += exp(s[j] - m);
            /* With n == 0 this is 0/0: NaN, as for an all -inf softmax row. */
            double l = (n > 0) ? m + log(denom) : NAN;
            if (lse) lse[b * H + h] = (n > 0) ? l : -INFINITY;

            /* Step 6 (mix): O~[c] = sum_t A_t * c_t[c], latent features only. */
            for (int64_t c = 0; c < Dc; ++c) mix[c] = 0.0;
            for (int64_t j = 0; j < n; ++j) {
                const double a = (n > 0) ? exp(s[j] - m) / denom : NAN;
                const double* crow = kv + b * kv_sb + set[j] * kv_st;
                for (int64_t c = 0; c < Dc; ++c) mix[c] += a * crow[c];
            }
            if (n == 0) for (int64_t c = 0; c < Dc; ++c) mix[c] = NAN;

            /* Step 7 (value-up): O[d] = sum_c O~[c] * W_UV[d][c]. */
            for (int64_t d = 0; d < Dv; ++d) {
                double acc = 0.0;
                for (int64_t c = 0; c < Dc; ++c) acc += mix[c] * w_uv[d * Dc + c];
                out[(b * H + h) * Dv + d] = acc;
            }
            if (q_abs) memcpy(q_abs + (b * H + h) * Dc, qa, sizeof(double) * (size_t)Dc);
            if (o_lat) memcpy(o_lat + (b * H + h) * Dc, mix, sizeof(double) * (size_t)Dc);

            /* Per-slot weights and scores, for the mask/normalisation checks. */
            if (indices && (weights || scores)) {
                const int64_t* row = indices + b * k_max;
                for (int64_t j = 0; j < k_max; ++j) {
                    double wv = 0.0, sv = -INFINITY;
                    if (row[j] >= 0) {
                        /* position of this slot inside the sorted set */
                        int64_t lo = 0, hi = n - 1, pos = -1;
                        while (lo <= hi) {
                            int64_t mid = (lo + hi) / 2;
                            if (set[mid] == row[j]) { pos = mid; break; }
                            if (set[mid] < row[j]) lo = mid + 1; else hi = mid - 1;
                        }
                        if (pos >= 0) { sv = s[pos]; wv = exp(s[pos] - m) / denom; }
                    }
                    if (weights) weights[(b * H + h) * k_max + j] = wv;
                    if (scores) scores[(b * H + h) * k_max + j] = sv;
                }
            }
            free(qa); free(s); free(mix);
        }
        free(set); free(mark);
    }
    return status;
}

/*
 * Step 2 alone ("Query-key similarity" page, code excerpt, absorption):
 *   q_abs[b][h][c] = sum_d q_nope[b][h][d] * W_UK,h[d][c]
 * q_nope [B][H][Dn]; wkv_b as in oracle_decode; q_abs [B][H][Dc].
 */
int oracle_absorb(int64_t B, int64_t H, int64_t Dn, int64_t Dc, int64_t Dv,
                  const double* q_nope, const double* wkv_b, double* q_abs) {
    if (B <= 0 || H <= 0 || Dn <= 0 || Dc <= 0 || Dv <= 0 || !q_nope || !wkv_b || !q_abs)
        return ORACLE_ERR_ARG;
    #pragma omp parallel for schedule(static)
    for (int64_t bh = 0; bh < B * H; ++bh) {
        const int64_t h = bh % H;
        const double* w_uk = wkv_b + (h * (Dn + Dv)) * Dc;
        for (int64_t c = 0; c < Dc; ++c) {
            double acc = 0.0;
            for (int64_t d = 0; d < Dn; ++d) acc += q_nope[bh * Dn + d] * w_uk[d * Dc + c];
            q_abs[bh * Dc + c] = acc;
        }
    }
    return ORACLE_OK;
}

/*
 * Step 7 alone ("Apply value weights" page, formula O_i = O~_i W_UV,i, with
 * W_UV,i the transpose of the stored [d][c] slice):
 *   out[b][h][d] = sum_c o_lat[b][h][c] * W_UV,h[d][c]
 */
int oracle_value_up(int64_t B, int64_t H, int64_t Dn, int64_t Dc, int64_t Dv,
                    const double* o_lat, const double* wkv_b, double* out) {
    if (B <= 0 || H <= 0 || Dn <= 0 || Dc <= 0 || Dv <= 0 || !o_lat || !wkv_b || !out)
        return ORACLE_ERR_ARG;
    #pragma omp parallel for schedule(static)
    for (int64_t bh = 0; bh < B * H; ++bh) {
        const int64_t h = bh % H;
        const double* w_uv = wkv_b + (h * (Dn + Dv) + Dn) * Dc;
        for (int64_t d = 0; d < Dv; ++d) {
            double acc = 0.0;
            for (int64_t c = 0; c < Dc; ++c) acc += o_lat[bh * Dc + c] * w_uv[d * Dc + c];
            out[bh * Dv + d] = acc;
        }
    }
    return ORACLE_OK;
}

/* Output projection ("Attention update" page, mla-output excerpt): each
 * sequence's head outputs flattened to one vector x[b][i] (i = h * Dv + d)
 * and projected to the model width by the output linear layer:
 * out[b][o] = sum_i x[b][i] * wo[o][i], with wo stored [Dout][Din] as a
 * linear layer's weight (no bias). */
int oracle_output_proj(int64_t B, int64_t Din, int64_t Dout, const double* x, const double* wo, double* out) {
    if (B <= 0 || Din <= 0 || Dout <= 0 || !x || !wo || !out) return ORACLE_ERR_ARG;
    #pragma omp parallel for schedule(static)
    for (int64_t bo = 0; bo < B * Dout; ++bo) {
        const int64_t b = bo / Dout, o = bo % Dout;
        double acc = 0.0;
        for (int64_t i = 0; i < Din; ++i) acc += x[b * Din + i] * wo[o * Din + i];
        out[bo] = acc;
    }
    return ORACLE_OK;
}

/*
 * Sparse prefill, the full-sequence (MHA) path ("Queries" page, prefill
 * mode, mla-prefill excerpt): the latent of every prompt position is
 * up-projected into per-head keys and values, each head's key joins its
 * non-rotary part with the shared rotary key, and the scores are scaled,
 * masked by the indexer's selection and the causal mask, normalised over the
 * keys and used to mix the values.  Keys are the prompt's own positions
 * 0 .. T-1 (the excerpt's start_pos = 0); query s may attend key t only if
 * t <= s (causal mask) and t is named in indices[b][s] (index mask, a
 * scatter of a constant: a set).  NULL indices select every causal key.
 *
 *   q_nope [B][T][H][Dn], q_pe [B][T][H][Dr]          (contiguous)
 *   kv: latent of (b, t) at kv + b*kv_sb + t*kv_st, Dc values
 *   pe: rotary key of (b, t) at pe + b*pe_sb + t*pe_st, Dr values
 *   wkv_b [H*(Dn+Dv)][Dc] as in oracle_decode
 *   indices [B][T][k_max] or NULL; -1 is padding; an index >= T or < -1 is
 *       an error; an index t > s is masked by causality.
 *   out [B][T][H][Dv], lse [B][T][H] (may be NULL),
 *   attended [B][T][T] (may be NULL): 1 where key t is attended by query s.
 */
int oracle_prefill(int64_t B, int64_t T, int64_t H, int64_t Dn, int64_t Dc, int64_t Dr,
                   int64_t Dv, const double* q_nope, const double* q_pe,
                   const double* kv, int64_t kv_sb, int64_t kv_st,
                   const double* pe, int64_t pe_sb, int64_t pe_st,
                   const double* wkv_b, const int64_t* indices, int64_t k_max,
                   double scale, double* out, double* lse, unsigned char* attended) {
    if (B <= 0 || T <= 0 || H <= 0 || Dn <= 0 || Dc <= 0 || Dr < 0 || Dv <= 0 ||
        !q_nope || !kv || !wkv_b || !out || (Dr > 0 && (!q_pe || !pe)))
        return ORACLE_ERR_ARG;
    if (indices && k_max <= 0) return ORACLE_ERR_ARG;
    if (indices)
        for (int64_t i = 0; i < B * T * k_max; ++i)
            if (indices[i] < -1 || indices[i] >= T) return ORACLE_ERR_INDEX_RANGE;
    int status = ORACLE_OK;
    for (int64_t b = 0; b < B; ++b) {
        /* The up-projection of every prompt position: k_nope[t][h][d] and
         * v[t][h][d] from the latent c_t (the excerpt's wkv_b(kv)). */
        double* knope = (double*)malloc(sizeof(double) * (size_t)(T * H * Dn));
        double* v = (double*)malloc(sizeof(double) * (size_t)(T * H * Dv));
        #pragma omp parallel for schedule(static)
        for (int64_t th = 0; th < T * H; ++th) {
            const int64_t t = th / H, h = th % H;
            const double* c = kv + b * kv_sb + t * kv_st;
            const double* w_uk = wkv_b + (h * (Dn + Dv)) * Dc;
            const double* w_uv = wkv_b + (h * (Dn + Dv) + Dn) * Dc;
            for (int64_t d = 0; d < Dn; ++d) {
                double acc = 0.0;
                for (int64_t j = 0; j < Dc; ++j) acc += w_uk[d * Dc + j] * c[j];
                knope[th * Dn + d] = acc;
            }
            for (int64_t d = 0; d < Dv; ++d) {
                double acc = 0.0;
                for (int64_t j = 0; j < Dc; ++j) acc += w_uv[d * Dc + j] * c[j];
                v[th * Dv + d] = acc;
            }
        }
        #pragma omp parallel for schedule(dynamic, 1) reduction(|:status)
        for (int64_t s = 0; s < T; ++s) {
            /* The attended keys of query s: selected and not in the future. */
            unsigned char* mark = (unsigned char*)calloc((size_t)T, 1);
            if (indices) {
                const int64_t* row = indices + (b * T + s) * k_max;
                for (int64_t j = 0; j < k_max; ++j)
                    if (row[j] >= 0 && row[j] <= s) mark[row[j]] = 1;
            } else {
                for (int64_t t = 0; t <= s; ++t) mark[t] = (unsigned char)1;
            }
            int64_t n = 0;
            for (int64_t t = 0; t < T; ++t) n += mark[t];
            if (n == 0) status |= ORACLE_ERR_EMPTY;
            if (attended) memcpy(attended + (b * T + s) * T, mark, (size_t)T);
            double* sc = (double*)malloc(sizeof(double) * (size_t)T);
            for (int64_t h = 0; h < H; ++h) {
                const double* qn = q_nope + ((b * T + s) * H + h) * Dn;
                const double* qr = Dr > 0 ? q_pe + ((b * T + s) * H + h) * Dr : NULL;
                /* scores over the keys [k_nope | k_pe] of this head, scaled */
                double m = -INFINITY;
                for (int64_t t = 0; t < T; ++t) {
                    if (!mark[t]) { sc[t] = -INFINITY; continue; }
                    const double* kn = knope + (t * H + h) * Dn;
                    double acc = 0.0;
                    for (int64_t d = 0; d < Dn; ++d) acc += qn[d] * kn[d];
                    if (Dr > 0) {
                        const double* kr = pe + b * pe_sb + t * pe_st;
                        for (int64_t r = 0; r < Dr; ++r) acc += qr[r] * kr[r];
                    }
                    sc[t] = acc * scale;
                    if (sc[t] > m) m = sc[t];
                }
                double denom = 0.0;
                for (int64_t t = 0; t < T; ++t) if (mark[t]) denom += exp(sc[t] - m);
                if (lse) lse[(b * T + s) * H + h] = n > 0 ? log(denom) + m : -INFINITY;
                double* o = out + ((b * T + s) * H + h) * Dv;
                for (int64_t d = 0; d < Dv; ++d) o[d] = 0.0;
                for (int64_t t = 0; t < T; ++t) {
                    if (!mark[t]) continue;
                    const double a = exp(sc[t] - m) / denom;
                    const double* vv = v + (t * H + h) * Dv;
                    for (int64_t d = 0; d < Dv; ++d) o[d] += a * vv[d];
                }
                if (n == 0) for (int64_t d = 0; d < Dv; ++d) o[d] = NAN;
            }
            free(sc);
            free(mark);
        }
        free(knope);
        free(v);
    }
    return status;
}
