/*
 * ep_oracle.c -- plain, slow, scalar CPU oracle for MoE token dispatch / combine.
 *
 * TEST INFRASTRUCTURE ONLY.  Nothing in the product path may link, load or call
 * this file.  Its only users are the tests under tests/, the smoke check in
 * __graft_entry__.py and the cpu_baseline leg of bench.py.  It shares no code,
 * header, table or constant generator with the HIP library.
 *
 * What it computes, and where that is defined
 * -------------------------------------------
 * The method: tokens pick top-k experts; dispatch sends each token's hidden
 * state to its experts, arranged by expert; combine brings the expert outputs
 * back to the original token order and reduces them with the routing weights.
 * Sources (web pages, cited by title and section):
 *   [yololab] "DeepEP是什麼？MoE Dispatch、Combine、All-to-all與V2架構",
 *             section "MoE為什麼需要All-to-all？" (stage table: dispatch takes
 *             tokens, top-k index and weights and yields hidden states arranged
 *             by expert; combine takes expert outputs and routing weights and
 *             yields results in the original token order), section
 *             "FP8與低精度通訊" (low-precision dispatch with scales; check the
 *             scale granularity and format), section "ElasticBuffer" (capacity
 *             headroom; overflow needs a drop policy), section "Load Imbalance"
 *             (per-expert token counts, per-rank send/receive volume).
 *   [backyes] "DeepEP 编址服务深度对抗分析", section 五.2 "MoE EP AllToAll 的
 *             特殊性" (dispatch and combine each move batch x top_k x hidden x
 *             sizeof(dtype): one receive row per (token, k) pair, no dedup).
 *   [donniechu] DeepEP v2 release notes, section "Số liệu kỹ thuật" (benchmark
 *             configuration: 8K tokens, hidden 7168, FP8 dispatch, BF16 combine).
 * Where the pages leave a step open, this file takes one plain reading; every
 * reading is named at the function that applies it (R1..R14 below).
 *
 * Readings
 *   R1  Order inside an expert's segment: stable in the flattened pair index
 *       p = t*k + j (a counting sort).  The pages fix no order.
 *   R2  topk_idx == -1 marks an unrouted pair: no slot, contributes nothing, no
 *       error.  Any other id outside [0, E) is treated the same way and sets
 *       error bit 0.
 *   R3  Experts map to G logical groups in contiguous blocks of E/G.
 *   R4  No per-group dedup: one receive row per valid (token, k) pair.
 *   R5  Padded mode (capacity > 0): expert e owns rows [e*cap, (e+1)*cap); a
 *       pair whose rank inside its expert is >= cap is dropped (slot -1) and
 *       sets error bit 1.  Counts stay unclamped (they report the demand).
 *   R6  FP8 is OCP E4M3 ("e4m3fn"): bias 7, largest finite 448, subnormals
 *       down to 2^-9, no infinities, 0x7F/0xFF are NaN.
 *   R7  One fp32 scale per (receive row, block of 128 channels):
 *       a = max(amax, 1e-4f); scale = a / 448 and inv = 448 / a, both single
 *       correctly rounded fp32 divisions.
 *   R8  Quantised code: v = x * inv (one fp32 multiply), clamped to
 *       [-448, 448], rounded to the nearest E4M3 value, ties to even; the
 *       sign is kept, so a negative value that rounds to zero encodes 0x80.
 *       Non-finite inputs (fp32-scale path): the block maximum skips NaN; a
 *       v that is NaN encodes 0x7F whatever its sign; a block holding an
 *       infinity has a = inf, so scale = inf, inv = +0, its finite values
 *       encode +-0 and its infinities (inf * 0 = NaN) 0x7F.
 *   R9  Scales are laid out row-major [R, H/128], one scale row per receive row.
 *   R10 Combine: out[t] = bf16(sum_j w[t,j] * y[slot[t,j]]), skipping dropped
 *       or unrouted pairs; no renormalisation.  The oracle sums in fp64 (each
 *       product of an fp32 weight and a bf16 value is exact there), then
 *       rounds once to bf16, nearest-even.  A token with no valid pair gives +0.
 *   R11 Identity expert stand-in (harness only, not part of the method): with
 *       FP8 dispatch the expert output is the dequantised receive row,
 *       bf16(decode(q) * scale), rounded once from the exact product.
 *   R12 Integer types: topk_idx int64; counts, offsets and slots int32.
 *   R13 Power-of-two scale variant: the smallest power of two s with
 *       448 * s >= a; codes from the exact rescale x / s.
 *   R14 FP8 combine variant: expert outputs as E4M3 codes + per-block fp32
 *       scales, decoded exactly inside the weighted sum.
 *   R15 Per-group dedup variant: a token goes once to every group holding at
 *       least one of its valid experts.  Its groups, in ascending order, are
 *       its entries (padded with -1 to kg = min(k, G)); receive rows are
 *       group-major and, inside a group, in ascending token order.
 *   R16 Receiver metadata of the dedup variant: the row of (t, g) carries
 *       t's top-k list masked to group g (other entries -1, weight 0).
 *   R17 Group combine of the dedup variant: the expert side has already
 *       weighted and summed its experts' outputs into one row per (t, g);
 *       out[t] = bf16(sum of t's group rows), unit weights, rounded once.
 *   R18 MXFP8 variant (the microscaling format gfx950's scaled matrix
 *       instructions consume): one E8M0 scale byte per block of 32 channels,
 *       from the OCP Microscaling (MX) v1.0 conversion: shared exponent
 *       floor(log2(amax)) - 8, clamped to [-127, 127] (-127 for an all-zero
 *       block); codes saturate at +-448.
 *   R19 FP16 I/O variant: fp16 rows are dispatched as a bit copy; the fp16
 *       combine rounds the exact weighted sum once to binary16, nearest-even,
 *       subnormals kept, overflow to infinity.
 *   R20 MN-major scale layout (the layout conversion that the FP8 section of
 *       the yololab page asks to check; two pages say the v2 buffer adopts a
 *       GEMM layout): the same scale entries, stored transposed, entry c of
 *       receive row r at c * R + r.
 *   R21 MXFP8 combine variant: expert outputs as E4M3 codes + one E8M0 byte
 *       per (row, 32-channel block) with value 2^(byte - 127) (byte 255 is
 *       NaN), decoded exactly inside the weighted sum.
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

#define EXPORT __attribute__((visibility("default")))

/* ------------------------------------------------------------------------- */
/* Status codes (the oracle's own; they mirror the meaning, not the source,   */
/* of the library's codes).                                                    */
/* ------------------------------------------------------------------------- */
#define ORACLE_OK 0
#define ORACLE_ERR_NULL (-1)
#define ORACLE_ERR_SHAPE (-2)

/* ------------------------------------------------------------------------- */
/* bf16 <-> real numbers                                                       */
/* ------------------------------------------------------------------------- */

/* A bf16 value is the upper half of an fp32 bit pattern. */
EXPORT double ep_oracle_bf16_to_double(uint16_t b) {
    uint32_t u = (uint32_t)b << 16;
    float f;
    memcpy(&f, &u, sizeof f);
    return (double)f;
}

/* The bf16 value nearest to v, ties to the even significand (IEEE 754
 * round-to-nearest-even applied to an 8-bit significand with the fp32
 * exponent range).  Written from the definition: find the quantum of v's
 * binade, round v/quantum to an integer with ties to even, scale back. */
EXPORT uint16_t ep_oracle_bf16_from_double(double v) {
    if (isnan(v)) return (uint16_t)(signbit(v) ? 0xFFC0u : 0x7FC0u);
    uint16_t sign = signbit(v) ? 0x8000u : 0u;
    double a = fabs(v);
    if (isinf(a)) return (uint16_t)(sign | 0x7F80u);
    if (a == 0.0) return sign;
    const double min_normal = ldexp(1.0, -126);
    double quantum;
    if (a < min_normal) {
        quantum = ldexp(1.0, -133);          /* subnormal spacing: 2^-126 / 2^7 */
    } else {
        int ex;
        frexp(a, &ex);                       /* a in [2^(ex-1), 2^ex) */
        quantum = ldexp(1.0, ex - 1 - 7);    /* 7 stored mantissa bits */
    }
    double n = a / quantum;                  /* exact: power-of-two scaling */
    double r = nearbyint(n);                 /* default mode: ties to even */
    double val = r * quantum;
    const double max_finite = ldexp(255.0, 127 - 7); /* (2 - 2^-7) * 2^127 */
    if (val > max_finite) return (uint16_t)(sign | 0x7F80u);
    float f = (float)val;                    /* exact: val is a bf16 value */
    uint32_t u;
    memcpy(&u, &f, sizeof u);
    return (uint16_t)(sign | (uint16_t)((u >> 16) & 0x7FFFu));
}

static float bf16_to_float(uint16_t b) {
    uint32_t u = (uint32_t)b << 16;
    float f;
    memcpy(&f, &u, sizeof f);
    return f;
}

/* ------------------------------------------------------------------------- */
/* OCP FP8 E4M3 (reading R6)                                                   */
/* ------------------------------------------------------------------------- */

/* Value of an E4M3 code from the format's definition. */
EXPORT double ep_oracle_e4m3_decode(uint8_t code) {
    int s = (code >> 7) & 1;
    int e = (code >> 3) & 0xF;
    int m = code & 7;
    if (e == 0xF && m == 7) return NAN;               /* the only NaN codes */
    double mag = (e == 0) ? ldexp((double)m, -9)       /* m/8 * 2^(1-7) */
                          : ldexp(1.0 + m / 8.0, e - 7);
    return s ? -mag : mag;
}

/* Magnitudes of the 127 non-negative finite codes 0x00..0x7E, ascending. */
static double g_e4m3_mag[127];
static int g_e4m3_ready = 0;

static void e4m3_table_init(void) {
    if (g_e4m3_ready) return;
    for (int c = 0; c < 127; ++c) g_e4m3_mag[c] = ep_oracle_e4m3_decode((uint8_t)c);
    g_e4m3_ready = 1;
}

/* Nearest E4M3 value to v, ties to the even code (the even significand);
 * magnitudes above 448 saturate to 448 (callers clamp first, reading R8);
 * the sign bit of v is kept; NaN encodes 0x7F. */
EXPORT uint8_t ep_oracle_e4m3_encode(float v) {
    e4m3_table_init();
    if (isnan(v)) return 0x7F;
    uint8_t sign = signbit(v) ? 0x80 : 0x00;
    double a = fabs((double)v);
    if (a >= g_e4m3_mag[126]) return (uint8_t)(sign | 126);
    /* largest code lo with mag[lo] <= a (binary search over the ascending table) */
    int lo = 0, hi = 126;
    while (hi - lo > 1) {
        int mid = (lo + hi) / 2;
        if (g_e4m3_mag[mid] <= a) lo = mid; else hi = mid;
    }
    /* now mag[lo] <= a < mag[lo+1] */
    double d_lo = a - g_e4m3_mag[lo];
    double d_hi = g_e4m3_mag[lo + 1] - a;
    int code;
    if (d_lo < d_hi) code = lo;
    else if (d_hi < d_lo) code = lo + 1;
    else code = (lo % 2 == 0) ? lo : lo + 1;          /* tie: even code */
    return (uint8_t)(sign | code);
}

EXPORT void ep_oracle_e4m3_encode_array(const float* v, int64_t n, uint8_t* out) {
    for (int64_t i = 0; i < n; ++i) out[i] = ep_oracle_e4m3_encode(v[i]);
}

/* Encode the n fp32 values whose bit patterns are first, first+1, ... */
EXPORT void ep_oracle_e4m3_encode_bits(uint32_t first, int64_t n, uint8_t* out) {
    for (int64_t i = 0; i < n; ++i) {
        uint32_t u = first + (uint32_t)i;
        float f;
        memcpy(&f, &u, sizeof f);
        out[i] = ep_oracle_e4m3_encode(f);
    }
}

/* ------------------------------------------------------------------------- */
/* Layout: per-expert counts, offsets, per-group counts, slot of every pair    */
/* ([yololab] stage table and "Load Imbalance"; readings R1-R5)                */
/* ------------------------------------------------------------------------- */

/* Number of receive rows: T*k in contiguous mode, E*cap in padded mode. */
EXPORT int64_t ep_oracle_num_recv_rows(int64_t T, int32_t k, int32_t E, int32_t cap) {
    return cap > 0 ? (int64_t)E * cap : T * (int64_t)k;
}

EXPORT int ep_oracle_layout(const int64_t* topk_idx, int64_t T, int32_t k, int32_t E,
                            int32_t G, int32_t cap, int32_t* num_tokens_per_expert,
                            int32_t* expert_offsets, int32_t* num_tokens_per_group,
                            int32_t* slot_idx, int32_t* recv_src, int32_t* error_flags) {
    if (T < 0 || k < 1 || E < 1 || G < 1 || cap < 0 || E % G != 0) return ORACLE_ERR_SHAPE;
    if ((T > 0 && (!topk_idx || !slot_idx)) || !num_tokens_per_expert || !expert_offsets ||
        !num_tokens_per_group || !error_flags)
        return ORACLE_ERR_NULL;
    int64_t P = T * (int64_t)k;
    int32_t flags = 0;

    /* 1. count the valid pairs of every expert */
    for (int32_t e = 0; e < E; ++e) num_tokens_per_expert[e] = 0;
    for (int64_t p = 0; p < P; ++p) {
        int64_t e = topk_idx[p];
        if (e == -1) continue;                        /* R2: unrouted */
        if (e < 0 || e >= E) { flags |= 1; continue; } /* R2: invalid id */
        num_tokens_per_expert[e] += 1;
    }

    /* 2. expert offsets: exclusive prefix sum (contiguous) or e*cap (padded, R5) */
    if (cap == 0) {
        expert_offsets[0] = 0;
        for (int32_t e = 0; e < E; ++e)
            expert_offsets[e + 1] = expert_offsets[e] + num_tokens_per_expert[e];
    } else {
        for (int32_t e = 0; e <= E; ++e) expert_offsets[e] = e * cap;
    }

    /* 3. per-group totals over contiguous expert blocks (R3) */
    int32_t per_group = E / G;
    for (int32_t g = 0; g < G; ++g) {
        int32_t s = 0;
        for (int32_t e = g * per_group; e < (g + 1) * per_group; ++e) s += num_tokens_per_expert[e];
        num_tokens_per_group[g] = s;
    }

    /* 4. slots: walk the pairs in p order with one running cursor per expert (R1) */
    int32_t* cursor = (int32_t*)calloc((size_t)E, sizeof(int32_t));
    if (!cursor) return ORACLE_ERR_NULL;
    for (int64_t p = 0; p < P; ++p) {
        int64_t e = topk_idx[p];
        if (e < 0 || e >= E) { slot_idx[p] = -1; continue; }
        int32_t r = cursor[e]++;
        if (cap > 0 && r >= cap) { slot_idx[p] = -1; flags |= 2; continue; } /* R5: drop */
        slot_idx[p] = expert_offsets[e] + r;
        if (recv_src) recv_src[slot_idx[p]] = (int32_t)p;
    }
    free(cursor);
    *error_flags = flags;
    return ORACLE_OK;
}

/* ------------------------------------------------------------------------- */
/* Dispatch ([yololab] stage table; [backyes] 五.2: one row per pair, R4)      */
/* ------------------------------------------------------------------------- */

/* bf16 dispatch: receive row slot[p] is a bit copy of token p/k's row. */
EXPORT void ep_oracle_dispatch_bf16(const uint16_t* x, int64_t T, int32_t k, int32_t H,
                                    const int32_t* slot_idx, uint16_t* recv_x) {
    for (int64_t p = 0; p < T * (int64_t)k; ++p) {
        int32_t s = slot_idx[p];
        if (s < 0) continue;
        int64_t t = p / k;
        for (int32_t c = 0; c < H; ++c) recv_x[(int64_t)s * H + c] = x[t * H + c];
    }
}

/* FP8 quantisation of one token row ([yololab] "FP8與低精度通訊"; R6-R8):
 * per block of 128 channels, scale from the block's largest magnitude, then
 * every channel to the nearest E4M3 code of x * inv. */
EXPORT void ep_oracle_quantize_token_fp8(const uint16_t* x_row, int32_t H, uint8_t* q_row,
                                         float* scales_row) {
    const int32_t B = 128;
    for (int32_t b = 0; b < H / B; ++b) {
        float amax = 0.0f;
        for (int32_t c = b * B; c < (b + 1) * B; ++c) {
            float m = fabsf(bf16_to_float(x_row[c]));
            if (m > amax) amax = m;
        }
        float a = amax > 1e-4f ? amax : 1e-4f;
        float scale = a / 448.0f;
        float inv = 448.0f / a;
        scales_row[b] = scale;
        for (int32_t c = b * B; c < (b + 1) * B; ++c) {
            float v = bf16_to_float(x_row[c]) * inv;
            if (v > 448.0f) v = 448.0f;
            if (v < -448.0f) v = -448.0f;
            q_row[c] = ep_oracle_e4m3_encode(v);
        }
    }
}

/* FP8 dispatch: every valid slot of token t receives t's codes and scales. */
EXPORT void ep_oracle_dispatch_fp8(const uint16_t* x, int64_t T, int32_t k, int32_t H,
                                   const int32_t* slot_idx, uint8_t* recv_q, float* recv_scales) {
    int32_t nb = H / 128;
    uint8_t* q = (uint8_t*)malloc((size_t)H);
    float* sc = (float*)malloc((size_t)nb * sizeof(float));
    if (!q || !sc) { free(q); free(sc); return; }
    for (int64_t t = 0; t < T; ++t) {
        ep_oracle_quantize_token_fp8(x + t * H, H, q, sc);
        for (int32_t j = 0; j < k; ++j) {
            int32_t s = slot_idx[t * k + j];
            if (s < 0) continue;
            memcpy(recv_q + (int64_t)s * H, q, (size_t)H);
            memcpy(recv_scales + (int64_t)s * nb, sc, (size_t)nb * sizeof(float));
        }
    }
    free(q);
    free(sc);
}

/* Identity expert stand-in for FP8 dispatch (harness only, R11). */
EXPORT void ep_oracle_dequant_fp8(const uint8_t* q, const float* scales, int64_t R, int32_t H,
                                  uint16_t* y) {
    int32_t nb = H / 128;
    for (int64_t r = 0; r < R; ++r)
        for (int32_t c = 0; c < H; ++c)
            y[r * H + c] = ep_oracle_bf16_from_double(ep_oracle_e4m3_decode(q[r * H + c]) *
                                                      (double)scales[r * nb + c / 128]);
}

/* ------------------------------------------------------------------------- */
/* Combine ([yololab] stage table, combine row; R10)                           */
/* ------------------------------------------------------------------------- */

static void combine_one(const uint16_t* y, const float* w, const int32_t* slot_idx, int64_t t,
                        int32_t k, int32_t H, uint16_t* out_row) {
    for (int32_t c = 0; c < H; ++c) {
        double acc = 0.0;
        for (int32_t j = 0; j < k; ++j) {
            int32_t s = slot_idx[t * k + j];
            if (s < 0) continue;
            acc += (double)w[t * k + j] * ep_oracle_bf16_to_double(y[(int64_t)s * H + c]);
        }
        out_row[c] = ep_oracle_bf16_from_double(acc);
    }
}

EXPORT void ep_oracle_combine(const uint16_t* y, const float* w, const int32_t* slot_idx,
                              int64_t T, int32_t k, int32_t H, uint16_t* out) {
    for (int64_t t = 0; t < T; ++t) combine_one(y, w, slot_idx, t, k, H, out + t * H);
}

/* Combine for a list of tokens only (for sampled checks at full size). */
EXPORT void ep_oracle_combine_tokens(const uint16_t* y, const float* w, const int32_t* slot_idx,
                                     int32_t k, int32_t H, const int64_t* tokens, int64_t n,
                                     uint16_t* out_rows) {
    for (int64_t i = 0; i < n; ++i) combine_one(y, w, slot_idx, tokens[i], k, H, out_rows + i * H);
}

/* ------------------------------------------------------------------------- */
/* Variants: power-of-two scales, FP8 combine                                  */
/* ([yololab] "FP8與低精度通訊": low precision cuts dispatch / combine volume;  */
/* the scale format is the implementation's to fix)                            */
/* ------------------------------------------------------------------------- */

/* R13 Power-of-two scales: a block's scale is the smallest power of two s
 * with 448 * s >= a, a = max(amax, 1e-4f); each code is the nearest E4M3
 * value of clamp(x / s, -448, 448), ties to even (x / s is an exact
 * power-of-two rescale). */
EXPORT void ep_oracle_quantize_token_fp8_pow2(const uint16_t* x_row, int32_t H, uint8_t* q_row,
                                              float* scales_row) {
    const int32_t B = 128;
    for (int32_t b = 0; b < H / B; ++b) {
        float amax = 0.0f;
        for (int32_t c = b * B; c < (b + 1) * B; ++c) {
            float m = fabsf(bf16_to_float(x_row[c]));
            if (m > amax) amax = m;
        }
        float a = amax > 1e-4f ? amax : 1e-4f;
        int e;
        frexp((double)a / 448.0, &e);                  /* a first guess */
        while (ldexp(448.0, e - 1) >= (double)a) --e;  /* exact comparisons */
        while (ldexp(448.0, e) < (double)a) ++e;
        scales_row[b] = (float)ldexp(1.0, e);
        for (int32_t c = b * B; c < (b + 1) * B; ++c) {
            double v = ldexp((double)bf16_to_float(x_row[c]), -e);
            if (v > 448.0) v = 448.0;
            if (v < -448.0) v = -448.0;
            q_row[c] = ep_oracle_e4m3_encode((float)v);
        }
    }
}

EXPORT void ep_oracle_dispatch_fp8_pow2(const uint16_t* x, int64_t T, int32_t k, int32_t H,
                                        const int32_t* slot_idx, uint8_t* recv_q,
                                        float* recv_scales) {
    int32_t nb = H / 128;
    uint8_t* q = (uint8_t*)malloc((size_t)H);
    float* sc = (float*)malloc((size_t)nb * sizeof(float));
    if (!q || !sc) { free(q); free(sc); return; }
    for (int64_t t = 0; t < T; ++t) {
        ep_oracle_quantize_token_fp8_pow2(x + t * H, H, q, sc);
        for (int32_t j = 0; j < k; ++j) {
            int32_t s = slot_idx[t * k + j];
            if (s < 0) continue;
            memcpy(recv_q + (int64_t)s * H, q, (size_t)H);
            memcpy(recv_scales + (int64_t)s * nb, sc, (size_t)nb * sizeof(float));
        }
    }
    free(q);
    free(sc);
}

/* R14 FP8 combine: the expert outputs arrive as E4M3 codes with one fp32
 * scale per (row, 128-channel block); out[t] = bf16(sum_j w[t,j] * decode(q)
 * * scale) over valid pairs, summed in fp64 (each product is exact there) and
 * rounded once, nearest-even. */
static void combine_fp8_one(const uint8_t* q, const float* scales, const float* w,
                            const int32_t* slot_idx, int64_t t, int32_t k, int32_t H,
                            uint16_t* out_row) {
    int32_t nb = H / 128;
    for (int32_t c = 0; c < H; ++c) {
        double acc = 0.0;
        for (int32_t j = 0; j < k; ++j) {
            int32_t s = slot_idx[t * k + j];
            if (s < 0) continue;
            acc += (double)w[t * k + j] * ep_oracle_e4m3_decode(q[(int64_t)s * H + c]) *
                   (double)scales[(int64_t)s * nb + c / 128];
        }
        out_row[c] = ep_oracle_bf16_from_double(acc);
    }
}

EXPORT void ep_oracle_combine_fp8(const uint8_t* q, const float* scales, const float* w,
                                  const int32_t* slot_idx, int64_t T, int32_t k, int32_t H,
                                  uint16_t* out) {
    for (int64_t t = 0; t < T; ++t) combine_fp8_one(q, scales, w, slot_idx, t, k, H, out + t * H);
}

EXPORT void ep_oracle_combine_fp8_tokens(const uint8_t* q, const float* scales, const float* w,
                                         const int32_t* slot_idx, int32_t k, int32_t H,
                                         const int64_t* tokens, int64_t n, uint16_t* out_rows) {
    for (int64_t i = 0; i < n; ++i)
        combine_fp8_one(q, scales, w, slot_idx, tokens[i], k, H, out_rows + i * H);
}

/* ------------------------------------------------------------------------- */
/* Variant: per-group dedup ([yololab] "Load Imbalance" lists the bytes each   */
/* rank sends and receives; [backyes] 五.2 gives the no-dedup volume; this     */
/* variant sends a token once per group instead of once per expert)            */
/* ------------------------------------------------------------------------- */

/* R15, R16.  Outputs (kg = min(k, G), Rg = T * kg rows at most):
 *   group_idx [T, kg]          t's groups, ascending, then -1
 *   num_tokens_per_group [G]   tokens that reach group g
 *   group_offsets [G+1]        exclusive prefix sum of those counts
 *   group_slot [T, kg]         receive row of entry i of token t, or -1
 *   recv_token [Rg]            source token of each used row (optional)
 *   recv_topk_idx [Rg, k]      t's expert ids masked to the row's group (optional)
 *   recv_topk_weights [Rg, k]  the matching weights, 0 elsewhere (optional)
 *   error_flags                bit 0: an expert id outside [-1, E)          */
EXPORT int ep_oracle_group_layout(const int64_t* topk_idx, const float* topk_weights, int64_t T,
                                  int32_t k, int32_t E, int32_t G, int32_t* group_idx,
                                  int32_t* num_tokens_per_group, int32_t* group_offsets,
                                  int32_t* group_slot, int32_t* recv_token,
                                  int64_t* recv_topk_idx, float* recv_topk_weights,
                                  unsigned char* is_token_in_group, int32_t* error_flags) {
    if (T < 0 || k < 1 || E < 1 || G < 1 || E % G != 0) return ORACLE_ERR_SHAPE;
    if ((T > 0 && (!topk_idx || !group_idx || !group_slot)) || !num_tokens_per_group ||
        !group_offsets || !error_flags || (recv_topk_weights && !topk_weights))
        return ORACLE_ERR_NULL;
    int32_t kg = k < G ? k : G;
    int32_t per_group = E / G;
    int32_t flags = 0;

    /* 1. which groups each token reaches */
    unsigned char* in_group = (unsigned char*)calloc((size_t)(T > 0 ? T : 1) * (size_t)G, 1);
    if (!in_group) return ORACLE_ERR_NULL;
    for (int64_t t = 0; t < T; ++t) {
        for (int32_t j = 0; j < k; ++j) {
            int64_t e = topk_idx[t * k + j];
            if (e == -1) continue;
            if (e < 0 || e >= E) { flags |= 1; continue; }
            in_group[t * G + e / per_group] = 1;
        }
    }

    /* 2. each token's groups in ascending order, padded with -1 */
    for (int64_t t = 0; t < T; ++t) {
        int32_t i = 0;
        for (int32_t g = 0; g < G; ++g)
            if (in_group[t * G + g]) group_idx[t * kg + i++] = g;
        while (i < kg) group_idx[t * kg + i++] = -1;
    }

    /* 3. per-group counts and their exclusive prefix sum */
    for (int32_t g = 0; g < G; ++g) {
        int32_t c = 0;
        for (int64_t t = 0; t < T; ++t) c += in_group[t * G + g];
        num_tokens_per_group[g] = c;
    }
    group_offsets[0] = 0;
    for (int32_t g = 0; g < G; ++g)
        group_offsets[g + 1] = group_offsets[g] + num_tokens_per_group[g];

    /* 4. rows: walk the tokens in order with one running cursor per group */
    int32_t* cursor = (int32_t*)calloc((size_t)G, sizeof(int32_t));
    if (!cursor) { free(in_group); return ORACLE_ERR_NULL; }
    for (int64_t t = 0; t < T; ++t) {
        for (int32_t i = 0; i < kg; ++i) {
            int32_t g = group_idx[t * kg + i];
            if (g < 0) { group_slot[t * kg + i] = -1; continue; }
            int32_t row = group_offsets[g] + cursor[g]++;
            group_slot[t * kg + i] = row;
            if (recv_token) recv_token[row] = (int32_t)t;

            /* 5. the row's copy of t's top-k list, masked to group g (R16) */
            for (int32_t j = 0; j < k; ++j) {
                int64_t e = topk_idx[t * k + j];
                int mine = e >= 0 && e < E && e / per_group == g;
                if (recv_topk_idx) recv_topk_idx[(int64_t)row * k + j] = mine ? e : -1;
                if (recv_topk_weights)
                    recv_topk_weights[(int64_t)row * k + j] = mine ? topk_weights[t * k + j] : 0.0f;
            }
        }
    }
    free(cursor);
    if (is_token_in_group && T > 0) memcpy(is_token_in_group, in_group, (size_t)T * (size_t)G);
    free(in_group);
    *error_flags = flags;
    return ORACLE_OK;
}

/* R17: out[t] = bf16(sum over i of z[group_slot[t, i]]), skipping -1 entries,
 * summed in fp64 in ascending i (ascending group) and rounded once,
 * nearest-even.  A token with no entry gives +0. */
static void combine_groups_one(const uint16_t* z, const int32_t* group_slot, int64_t t,
                               int32_t kg, int32_t H, uint16_t* out_row) {
    for (int32_t c = 0; c < H; ++c) {
        double acc = 0.0;
        for (int32_t i = 0; i < kg; ++i) {
            int32_t r = group_slot[t * kg + i];
            if (r < 0) continue;
            acc += ep_oracle_bf16_to_double(z[(int64_t)r * H + c]);
        }
        out_row[c] = ep_oracle_bf16_from_double(acc);
    }
}

EXPORT void ep_oracle_combine_groups(const uint16_t* z, const int32_t* group_slot, int64_t T,
                                     int32_t kg, int32_t H, uint16_t* out) {
    for (int64_t t = 0; t < T; ++t) combine_groups_one(z, group_slot, t, kg, H, out + t * H);
}

EXPORT void ep_oracle_combine_groups_tokens(const uint16_t* z, const int32_t* group_slot,
                                            int32_t kg, int32_t H, const int64_t* tokens,
                                            int64_t n, uint16_t* out_rows) {
    for (int64_t i = 0; i < n; ++i)
        combine_groups_one(z, group_slot, tokens[i], kg, H, out_rows + i * H);
}

/* ------------------------------------------------------------------------- */
/* Variants: MXFP8 dispatch and FP16 I/O ([yololab] "FP8與低精度通訊": check   */
/* the scale's granularity and format; "Benchmark矩陣": BF16, FP16 and FP8)    */
/* ------------------------------------------------------------------------- */

/* R18.  Per block of 32 channels: amax = largest |x|; the shared exponent is
 * se = floor(log2(amax)) - 8, where 8 is the exponent of E4M3's largest
 * normal (448 = 1.75 * 2^8), clamped to [-127, 127]; an all-zero block takes
 * -127.  The block's scale byte is se + 127 (E8M0: the value 2^se).  Each
 * code is the nearest E4M3 value of clamp(x / 2^se, -448, 448), ties to even
 * (x / 2^se is an exact power-of-two rescale; amax / 2^se lies in [256, 512),
 * so the block's largest values may saturate at 448). */
EXPORT void ep_oracle_quantize_token_mxfp8(const uint16_t* x_row, int32_t H, uint8_t* q_row,
                                           uint8_t* scale_row) {
    const int32_t B = 32;
    for (int32_t b = 0; b < H / B; ++b) {
        double amax = 0.0;
        for (int32_t c = b * B; c < (b + 1) * B; ++c) {
            double m = fabs(ep_oracle_bf16_to_double(x_row[c]));
            if (m > amax) amax = m;
        }
        int se = -127;
        if (amax > 0.0) {
            int e;
            frexp(amax, &e);             /* amax in [2^(e-1), 2^e): floor(log2) = e - 1 */
            se = (e - 1) - 8;
            if (se < -127) se = -127;
            if (se > 127) se = 127;
        }
        scale_row[b] = (uint8_t)(se + 127);
        for (int32_t c = b * B; c < (b + 1) * B; ++c) {
            double v = ldexp(ep_oracle_bf16_to_double(x_row[c]), -se);
            if (v > 448.0) v = 448.0;
            if (v < -448.0) v = -448.0;
            q_row[c] = ep_oracle_e4m3_encode((float)v);
        }
    }
}

EXPORT void ep_oracle_dispatch_mxfp8(const uint16_t* x, int64_t T, int32_t k, int32_t H,
                                     const int32_t* slot_idx, uint8_t* recv_q,
                                     uint8_t* recv_scales) {
    int32_t nb = H / 32;
    uint8_t* q = (uint8_t*)malloc((size_t)H);
    uint8_t* sc = (uint8_t*)malloc((size_t)nb);
    if (!q || !sc) { free(q); free(sc); return; }
    for (int64_t t = 0; t < T; ++t) {
        ep_oracle_quantize_token_mxfp8(x + t * H, H, q, sc);
        for (int32_t j = 0; j < k; ++j) {
            int32_t s = slot_idx[t * k + j];
            if (s < 0) continue;
            memcpy(recv_q + (int64_t)s * H, q, (size_t)H);
            memcpy(recv_scales + (int64_t)s * nb, sc, (size_t)nb);
        }
    }
    free(q);
    free(sc);
}

/* Identity expert stand-in for MXFP8 rows (harness only): the bf16 nearest to
 * decode(q) * 2^(byte - 127), rounded once from the exact product; scale byte
 * 255 (which dispatch never writes) is NaN in E8M0 and gives the quiet NaN
 * 0x7FC0 for its whole block. */
EXPORT void ep_oracle_dequant_mxfp8(const uint8_t* q, const uint8_t* scales, int64_t R, int32_t H,
                                    uint16_t* y) {
    int32_t nb = H / 32;
    for (int64_t r = 0; r < R; ++r)
        for (int32_t c = 0; c < H; ++c) {
            uint8_t b = scales[r * nb + c / 32];
            if (b == 255) { y[r * H + c] = 0x7FC0u; continue; }
            double x = ldexp(1.0, (int)b - 127);                         /* E8M0: 2^(byte-127) */
            y[r * H + c] = ep_oracle_bf16_from_double(ep_oracle_e4m3_decode(q[r * H + c]) * x);
        }
}

/* fp16 (IEEE 754 binary16: 1 sign bit, 5 exponent bits with bias 15, 10
 * stored significand bits) -> real number. */
EXPORT double ep_oracle_f16_to_double(uint16_t h) {
    int sign = h >> 15;
    int e = (h >> 10) & 0x1F;
    int m = h & 0x3FF;
    double v;
    if (e == 0) v = ldexp((double)m, -24);                  /* subnormal: m * 2^-14 / 2^10 */
    else if (e == 31) v = m ? NAN : INFINITY;
    else v = ldexp(1024.0 + m, e - 15 - 10);
    return sign ? -v : v;
}

/* The binary16 value nearest to v, ties to even; magnitudes that round past
 * the largest finite value 65504 become infinity (the default IEEE rounding).
 * From the definition, as for bf16: the quantum of v's binade, an integer
 * rounding with ties to even, scaled back. */
EXPORT uint16_t ep_oracle_f16_from_double(double v) {
    if (isnan(v)) return (uint16_t)(signbit(v) ? 0xFE00u : 0x7E00u);
    uint16_t sign = signbit(v) ? 0x8000u : 0u;
    double a = fabs(v);
    if (isinf(a)) return (uint16_t)(sign | 0x7C00u);
    if (a == 0.0) return sign;
    double quantum;
    if (a < ldexp(1.0, -14)) {
        quantum = ldexp(1.0, -24);           /* subnormal spacing: 2^-14 / 2^10 */
    } else {
        int ex;
        frexp(a, &ex);                       /* a in [2^(ex-1), 2^ex) */
        quantum = ldexp(1.0, ex - 1 - 10);   /* 10 stored significand bits */
    }
    double r = nearbyint(a / quantum) * quantum;   /* ties to even */
    if (r > 65504.0) return (uint16_t)(sign | 0x7C00u);
    if (r < ldexp(1.0, -14)) return (uint16_t)(sign | (uint16_t)(r / ldexp(1.0, -24)));
    int ex;
    double m = frexp(r, &ex);                /* r = m * 2^ex, m in [0.5, 1) */
    uint16_t bits = (uint16_t)(((ex - 1 + 15) << 10) | (uint16_t)(ldexp(m, 11) - 1024.0));
    return (uint16_t)(sign | bits);
}

/* R19 fp16 combine: out[t] = f16(sum_j w[t,j] * y[slot[t,j]]) over valid
 * pairs, each product exact in fp64 (24 + 11 significand bits), the sum in
 * fp64, rounded once; +0 for a token with no valid pair. */
static void combine_f16_one(const uint16_t* y, const float* w, const int32_t* slot_idx, int64_t t,
                            int32_t k, int32_t H, uint16_t* out_row) {
    for (int32_t c = 0; c < H; ++c) {
        double acc = 0.0;
        for (int32_t j = 0; j < k; ++j) {
            int32_t s = slot_idx[t * k + j];
            if (s < 0) continue;
            acc += (double)w[t * k + j] * ep_oracle_f16_to_double(y[(int64_t)s * H + c]);
        }
        out_row[c] = ep_oracle_f16_from_double(acc);
    }
}

EXPORT void ep_oracle_combine_f16(const uint16_t* y, const float* w, const int32_t* slot_idx,
                                  int64_t T, int32_t k, int32_t H, uint16_t* out) {
    for (int64_t t = 0; t < T; ++t) combine_f16_one(y, w, slot_idx, t, k, H, out + t * H);
}

EXPORT void ep_oracle_combine_f16_tokens(const uint16_t* y, const float* w, const int32_t* slot_idx,
                                         int32_t k, int32_t H, const int64_t* tokens, int64_t n,
                                         uint16_t* out_rows) {
    for (int64_t i = 0; i < n; ++i)
        combine_f16_one(y, w, slot_idx, tokens[i], k, H, out_rows + i * H);
}

/* R20: row-major scale entries [rows, entries] of entry_bytes bytes each
 * (4 for fp32 scales, 1 for E8M0 bytes) -> MN-major [entries, rows]. */
EXPORT void ep_oracle_scales_mn_major(const uint8_t* src, int64_t rows, int32_t entries,
                                      int32_t entry_bytes, uint8_t* dst) {
    for (int64_t r = 0; r < rows; ++r)
        for (int32_t c = 0; c < entries; ++c)
            memcpy(dst + ((int64_t)c * rows + r) * entry_bytes,
                   src + (r * entries + c) * entry_bytes, (size_t)entry_bytes);
}

/* R21: an E8M0 scale byte's value, 2^(byte - 127); 255 encodes NaN (OCP MX). */
static double e8m0_value(uint8_t b) { return b == 255 ? NAN : ldexp(1.0, (int)b - 127); }

/* R21 MXFP8 combine: out[t] = bf16(sum_j w[t,j] * decode(q) * 2^(byte - 127))
 * over valid pairs, with one scale byte per (row, 32-channel block), summed in
 * fp64 (each product is exact there) and rounded once, nearest-even; +0 for a
 * token with no valid pair. */
static void combine_mxfp8_one(const uint8_t* q, const uint8_t* scales, const float* w,
                              const int32_t* slot_idx, int64_t t, int32_t k, int32_t H,
                              uint16_t* out_row) {
    int32_t nb = H / 32;
    for (int32_t c = 0; c < H; ++c) {
        double acc = 0.0;
        for (int32_t j = 0; j < k; ++j) {
            int32_t s = slot_idx[t * k + j];
            if (s < 0) continue;
            acc += (double)w[t * k + j] * ep_oracle_e4m3_decode(q[(int64_t)s * H + c]) *
                   e8m0_value(scales[(int64_t)s * nb + c / 32]);
        }
        out_row[c] = ep_oracle_bf16_from_double(acc);
    }
}

EXPORT void ep_oracle_combine_mxfp8(const uint8_t* q, const uint8_t* scales, const float* w,
                                    const int32_t* slot_idx, int64_t T, int32_t k, int32_t H,
                                    uint16_t* out) {
    for (int64_t t = 0; t < T; ++t) combine_mxfp8_one(q, scales, w, slot_idx, t, k, H, out + t * H);
}

EXPORT void ep_oracle_combine_mxfp8_tokens(const uint8_t* q, const uint8_t* scales, const float* w,
                                           const int32_t* slot_idx, int32_t k, int32_t H,
                                           const int64_t* tokens, int64_t n, uint16_t* out_rows) {
    for (int64_t i = 0; i < n; ++i)
        combine_mxfp8_one(q, scales, w, slot_idx, tokens[i], k, H, out_rows + i * H);
}
