/*
 * ep_oracle.c -- plain, slow CPU oracle for one GPU's share of MoE
 * expert-parallel dispatch and combine.
 *
 * TEST INFRASTRUCTURE ONLY.  Only the test suite, the smoke check and the
 * CPU-baseline leg of the benchmark may load or call this file.  It shares no
 * source, header, table or helper with the HIP library, and the HIP library
 * never calls it.
 *
 * Every function is the plain definition of what the pages describe, written
 * as straight scalar loops in the order the definition reads:
 *   - StreamEP README, "Streaming dispatch in one paragraph": the expert-major,
 *     BLOCK_M-padded pool; expert e's block starts at
 *     expert_pool_block_offset[e] * tile_m rows; every slot belongs to one
 *     expert and one tile; pool_arrival_target per tile; pool_recv_token >= 0
 *     marks real rows.
 *   - "DeepEP MoE dispatch/combine" blog, section on one DeepEP round (count
 *     per expert, layout and offsets, grouped receive, combine restores the
 *     source token / top-k slot) and section on router weights (the weighted
 *     sum y_t = sum_j p_{t,j} o_{t,j}).
 *   - instagit DeepEP low-latency page, "FP8 and Quantization Support":
 *     float8_e4m3fn payload with UE8M0 (power-of-two) scales.
 *
 * Build: gcc -O2 -ffp-contract=off -std=c11 -shared -fPIC (no fast-math), so
 * that fmaf is a single correctly rounded fused multiply-add and no other
 * expression is contracted.
 *
 * Readings where the pages are silent:
 *   - rows of one expert are filled in ascending flat slot order s = t*K + k;
 *   - topk id -1 is a masked slot; ids outside [-1, E) set error bit 1 and are
 *     treated as masked;
 *   - offsets are in tiles, E+1 entries, the last one is num_tiles;
 *   - tiles in [num_tiles, max_tiles) get tile_expert = -1 and target 0;
 *   - combine: fp32 accumulator from +0, fmaf in ascending k over unmasked
 *     slots, one round-to-nearest-even to bf16 at the end;
 *   - UE8M0 scale 2^e with e the smallest integer in [-127, 127] such that
 *     amax <= 448 * 2^e (e = 127 when none is), byte e + 127;
 *   - e4m3fn code = nearest finite code to |v|, ties to the even code, sign
 *     kept (-0 -> 0x80); |v| >= 448 gives 0x7E (only reachable from an
 *     infinite input), NaN gives 0x7F;
 *   - float32 scales (no UE8M0): amax floored at 448 * 2^-126, s = amax/448,
 *     codes of float(x * (448/amax)), see eo_quantize_row_f32scale.
 */
#include <math.h>
#include <stdint.h>
#include <string.h>

/* ---------------------------------------------------------------- bf16 --- */

/* bf16 bits -> float: the bf16 pattern is the top half of the binary32. */
float eo_bf16_to_f32(uint16_t b)
{
    uint32_t u = (uint32_t)b << 16;
    float f;
    memcpy(&f, &u, sizeof f);
    return f;
}

/* float -> bf16, round to nearest, ties to even.  Written as "pick the nearer
 * of the two neighbouring bf16 patterns", with the even one on a tie.  NaN
 * becomes the canonical quiet NaN 0x7FC0 (sign kept). */
uint16_t eo_f32_to_bf16(float f)
{
    uint32_t u;
    memcpy(&u, &f, sizeof u);
    if (isnan(f))
        return (uint16_t)(((u >> 16) & 0x8000u) | 0x7FC0u);
    uint32_t below = u >> 16;           /* truncated pattern */
    uint32_t rest = u & 0xFFFFu;        /* discarded half */
    int up;
    if (rest > 0x8000u)
        up = 1;
    else if (rest < 0x8000u)
        up = 0;
    else
        up = (int)(below & 1u);         /* exact tie: go to the even pattern */
    return (uint16_t)(below + (uint32_t)up);
}

/* ------------------------------------------------------------- e4m3fn --- */

/* Value of a non-negative OCP e4m3fn code 0x00..0x7E: sign-less, exponent
 * bias 7, 3 mantissa bits; exponent field 0 is subnormal (m * 2^-9). */
double eo_e4m3_value(int code)
{
    int ef = (code >> 3) & 0xF;
    int m = code & 7;
    if (ef == 0)
        return ldexp((double)m, -9);
    return ldexp(1.0 + (double)m / 8.0, ef - 7);
}

/* Nearest e4m3fn code to v, ties to the even code, by searching the ordered
 * table of finite magnitudes (codes 0x00..0x7E are increasing in value). */
uint8_t eo_e4m3_encode(double v)
{
    uint8_t sign = signbit(v) ? 0x80 : 0x00;
    if (isnan(v))
        return (uint8_t)(sign | 0x7F);
    double a = fabs(v);
    if (a >= 448.0)
        return (uint8_t)(sign | 0x7E);
    /* largest code lo with value(lo) <= a */
    int lo = 0, hi = 0x7E;
    while (lo < hi) {
        int mid = (lo + hi + 1) / 2;
        if (eo_e4m3_value(mid) <= a)
            lo = mid;
        else
            hi = mid - 1;
    }
    int code = lo;
    if (lo < 0x7E) {
        double dlo = a - eo_e4m3_value(lo);
        double dhi = eo_e4m3_value(lo + 1) - a;
        if (dhi < dlo || (dhi == dlo && ((lo + 1) % 2 == 0)))
            code = lo + 1;
    }
    return (uint8_t)(sign | (uint8_t)code);
}

/* UE8M0 exponent of a 128-channel group: the smallest e in [-127, 127] with
 * amax <= 448 * 2^e; 127 when no e qualifies (infinite amax). */
int eo_ue8m0_exponent(float amax)
{
    for (int e = -127; e <= 127; ++e)
        if ((double)amax <= ldexp(448.0, e))
            return e;
    return 127;
}

/* Quantise one token row of H bf16 values (H % 128 == 0) into H e4m3fn
 * bytes and H/128 UE8M0 scale bytes. */
void eo_quantize_row(const uint16_t* x, int32_t H, uint8_t* q, uint8_t* scales)
{
    for (int32_t g = 0; g < H / 128; ++g) {
        float amax = 0.0f;
        for (int c = 0; c < 128; ++c) {
            float a = fabsf(eo_bf16_to_f32(x[g * 128 + c]));
            if (a > amax)                /* NaN never compares greater */
                amax = a;
        }
        int e = eo_ue8m0_exponent(amax);
        scales[g] = (uint8_t)(e + 127);
        for (int c = 0; c < 128; ++c) {
            double v = (double)eo_bf16_to_f32(x[g * 128 + c]);
            q[g * 128 + c] = eo_e4m3_encode(ldexp(v, -e));
        }
    }
}

/* Inverse of the quantisation for one pool row: bf16(value(q) * 2^e).
 * This is the per_token_cast_back step of the low-latency example. */
void eo_dequant_row(const uint8_t* q, const uint8_t* scales, int32_t H, uint16_t* out)
{
    for (int32_t c = 0; c < H; ++c) {
        int e = (int)scales[c / 128] - 127;
        uint8_t b = q[c];
        double v = eo_e4m3_value(b & 0x7F);
        if ((b & 0x7F) == 0x7F)
            v = NAN;
        if (b & 0x80)
            v = -v;
        out[c] = eo_f32_to_bf16((float)ldexp(v, e));
    }
}

/* -------------------------------------------------------------- layout --- */

/* Stable bucket sort of the T*K routing slots by expert, each bucket padded
 * to a multiple of BM rows.  Returns the number of pool rows P in use, or -1
 * when the capacity given is too small (cannot happen for cap >= T*K +
 * E*(BM-1)).  Outputs:
 *   counts[E], offsets[E+1] (tiles), *num_tiles,
 *   tile_expert[max_tiles], tile_target[max_tiles],
 *   slot_to_row[T*K] (-1 for masked), recv_token[cap] (-1 for padding),
 *   *error |= 1 for ids outside [-1, E). */
int64_t eo_layout(const int32_t* idx, int64_t T, int32_t K, int32_t E, int32_t BM,
                  int64_t cap, int32_t max_tiles,
                  int32_t* counts, int32_t* offsets, int32_t* num_tiles,
                  int32_t* tile_expert, int32_t* tile_target,
                  int32_t* slot_to_row, int32_t* recv_token, int32_t* error)
{
    int64_t S = T * (int64_t)K;
    /* 1. count per expert */
    for (int32_t e = 0; e < E; ++e)
        counts[e] = 0;
    for (int64_t s = 0; s < S; ++s) {
        int32_t e = idx[s];
        if (e == -1)
            continue;
        if (e < -1 || e >= E) {
            *error |= 1;
            continue;
        }
        counts[e] += 1;
    }
    /* 2. tiles per expert and their exclusive prefix sum */
    offsets[0] = 0;
    for (int32_t e = 0; e < E; ++e) {
        int32_t tiles = (counts[e] + BM - 1) / BM;
        offsets[e + 1] = offsets[e] + tiles;
    }
    *num_tiles = offsets[E];
    if ((int64_t)offsets[E] * BM > cap || offsets[E] > max_tiles)
        return -1;
    /* 3. per-tile expert and arrival target */
    for (int32_t j = 0; j < max_tiles; ++j) {
        tile_expert[j] = -1;
        tile_target[j] = 0;
    }
    for (int32_t e = 0; e < E; ++e) {
        for (int32_t j = 0; j < offsets[e + 1] - offsets[e]; ++j) {
            int32_t left = counts[e] - j * BM;
            tile_expert[offsets[e] + j] = e;
            tile_target[offsets[e] + j] = left < BM ? left : BM;
        }
    }
    /* 4. everything starts unmapped */
    for (int64_t r = 0; r < cap; ++r)
        recv_token[r] = -1;
    for (int64_t s = 0; s < S; ++s)
        slot_to_row[s] = -1;
    /* 5. fill each expert's block in ascending slot order */
    for (int32_t e = 0; e < E; ++e) {
        int64_t next = (int64_t)offsets[e] * BM;
        for (int64_t s = 0; s < S; ++s) {
            if (idx[s] != e)
                continue;
            slot_to_row[s] = (int32_t)next;
            recv_token[next] = (int32_t)(s / K);
            next += 1;
        }
    }
    return (int64_t)offsets[E] * BM;
}

/* ------------------------------------------------------------ dispatch --- */

/* bf16 dispatch: every real pool row is a bitwise copy of its source token's
 * row of x; padding rows are left as they were. */
void eo_dispatch_bf16(const uint16_t* x, int32_t H, const int32_t* recv_token, int64_t cap,
                      uint16_t* pool)
{
    for (int64_t r = 0; r < cap; ++r) {
        int32_t t = recv_token[r];
        if (t < 0)
            continue;
        for (int32_t c = 0; c < H; ++c)
            pool[r * H + c] = x[(int64_t)t * H + c];
    }
}

/* FP8 dispatch: every real pool row holds the e4m3fn quantisation of its
 * source token's row, with that row's UE8M0 scales. */
void eo_dispatch_fp8(const uint16_t* x, int32_t H, const int32_t* recv_token, int64_t cap,
                     uint8_t* pool, uint8_t* scales)
{
    for (int64_t r = 0; r < cap; ++r) {
        int32_t t = recv_token[r];
        if (t < 0)
            continue;
        eo_quantize_row(x + (int64_t)t * H, H, pool + r * H, scales + r * (H / 128));
    }
}

/* ------------------------------------------------------------- combine --- */

/* y[t, c] = bf16( sum over unmasked k, in ascending k, of w[t,k] * o[row(t,k), c] )
 * with an fp32 accumulator starting at +0 and fmaf for every term. */
void eo_combine(const uint16_t* expert_out, int32_t H, const int32_t* slot_to_row,
                const float* w, int64_t T, int32_t K, uint16_t* y)
{
    for (int64_t t = 0; t < T; ++t) {
        for (int32_t c = 0; c < H; ++c) {
            float acc = 0.0f;
            for (int32_t k = 0; k < K; ++k) {
                int32_t r = slot_to_row[t * K + k];
                if (r < 0)
                    continue;
                acc = fmaf(w[t * K + k], eo_bf16_to_f32(expert_out[(int64_t)r * H + c]), acc);
            }
            y[t * H + c] = eo_f32_to_bf16(acc);
        }
    }
}

/* Combine for a chosen subset of tokens (sampled checks at full size): the
 * caller passes the K expert rows of each sampled token already gathered,
 * rows_of[i*K + k] (H values each), and a per-slot validity flag. */
void eo_combine_gathered(const uint16_t* rows_of, const int32_t* valid, const float* w,
                         int64_t n, int32_t K, int32_t H, uint16_t* y)
{
    for (int64_t i = 0; i < n; ++i) {
        for (int32_t c = 0; c < H; ++c) {
            float acc = 0.0f;
            for (int32_t k = 0; k < K; ++k) {
                if (!valid[i * K + k])
                    continue;
                acc = fmaf(w[i * K + k], eo_bf16_to_f32(rows_of[(i * K + k) * (int64_t)H + c]), acc);
            }
            y[i * H + c] = eo_f32_to_bf16(acc);
        }
    }
}

/* --------------------------------------------- array forms for testing --- */

void eo_e4m3_encode_n(const double* v, int64_t n, uint8_t* out)
{
    for (int64_t i = 0; i < n; ++i)
        out[i] = eo_e4m3_encode(v[i]);
}

void eo_f32_to_bf16_n(const float* f, int64_t n, uint16_t* out)
{
    for (int64_t i = 0; i < n; ++i)
        out[i] = eo_f32_to_bf16(f[i]);
}

void eo_ue8m0_exponent_n(const float* amax, int64_t n, int32_t* out)
{
    for (int64_t i = 0; i < n; ++i)
        out[i] = eo_ue8m0_exponent(amax[i]);
}

/* ------------------------------------------------------------ backward --- */

/* Backward of the combine (StreamEP README, "What's in the box": the buffer
 * exposes combine_grads for the backward pass; the pages give no formula, so
 * this is the derivative of y_t = sum_k w_{t,k} o_{row(t,k)}):
 *   grad_eo[row(t,k), c] = bf16( fp32( w[t,k] * grad_y[t,c] ) )
 *   grad_w[t,k]          = fp32( sum over c ascending of grad_y[t,c] * o[row,c] )
 *                          accumulated in double (each bf16 x bf16 product is
 *                          exact in double), rounded once to float
 * Masked slots: grad_w = 0 and no row is written. */
void eo_combine_backward(const uint16_t* grad_y, const uint16_t* expert_out,
                         const int32_t* slot_to_row, const float* w, int64_t T, int32_t K,
                         int32_t H, uint16_t* grad_eo, float* grad_w)
{
    for (int64_t t = 0; t < T; ++t) {
        for (int32_t k = 0; k < K; ++k) {
            int32_t r = slot_to_row[t * K + k];
            if (r < 0) {
                grad_w[t * K + k] = 0.0f;
                continue;
            }
            double dot = 0.0;
            for (int32_t c = 0; c < H; ++c) {
                float g = eo_bf16_to_f32(grad_y[t * H + c]);
                float o = eo_bf16_to_f32(expert_out[(int64_t)r * H + c]);
                float p = w[t * K + k] * g;
                grad_eo[(int64_t)r * H + c] = eo_f32_to_bf16(p);
                dot += (double)g * (double)o;
            }
            grad_w[t * K + k] = (float)dot;
        }
    }
}

/* Backward of the dispatch (dispatch_grads): every pool row was a copy of its
 * token's row, so the token's gradient is the sum of its rows' gradients:
 *   grad_x[t, c] = bf16( fp32 sum over unmasked k ascending of grad_pool[row(t,k), c] )
 * starting from +0; a token with no unmasked slot gets +0. */
void eo_dispatch_backward(const uint16_t* grad_pool, const int32_t* slot_to_row, int64_t T,
                          int32_t K, int32_t H, uint16_t* grad_x)
{
    for (int64_t t = 0; t < T; ++t) {
        for (int32_t c = 0; c < H; ++c) {
            float acc = 0.0f;
            for (int32_t k = 0; k < K; ++k) {
                int32_t r = slot_to_row[t * K + k];
                if (r < 0)
                    continue;
                acc = acc + eo_bf16_to_f32(grad_pool[(int64_t)r * H + c]);
            }
            grad_x[t * H + c] = eo_f32_to_bf16(acc);
        }
    }
}

/* ------------------------------------------------- FP8 with fp32 scales --- */

/* Quantisation with a float32 scale per 128-channel group: the use_ue8m0 =
 * false, round_scale = false flavour of the instagit page ("API Signature and
 * Return Values", "FP8 and Quantization Support").  The pages give no rule;
 * the reading is the usual amax scaling, all in float32:
 *   a      = max(amax, 448 * 2^-126)   (keeps s a normal float, f finite)
 *   s      = a / 448                   (the stored scale; x ~ value(q) * s)
 *   f      = 448 / a                   (the quantisation factor)
 *   q      = nearest e4m3fn code of float(x * f), ties to even, saturating
 *            at 448; a NaN product (NaN x, or infinite x times f = 0) gives
 *            0x7F with the sign of x. */
void eo_quantize_row_f32scale(const uint16_t* x, int32_t H, uint8_t* q, float* scales)
{
    const float floor_amax = 448.0f * 0x1p-126f;
    for (int32_t g = 0; g < H / 128; ++g) {
        float amax = 0.0f;
        for (int c = 0; c < 128; ++c) {
            float a = fabsf(eo_bf16_to_f32(x[g * 128 + c]));
            if (a > amax)                /* NaN never compares greater */
                amax = a;
        }
        float a = amax > floor_amax ? amax : floor_amax;
        float s = a / 448.0f;
        float f = 448.0f / a;
        scales[g] = s;
        for (int c = 0; c < 128; ++c) {
            float xv = eo_bf16_to_f32(x[g * 128 + c]);
            float v = xv * f;
            uint8_t code;
            if (isnan(v))
                code = 0x7F;
            else
                code = eo_e4m3_encode(fabs((double)v));
            if (signbit(xv))
                code |= 0x80;
            q[g * 128 + c] = code;
        }
    }
}

/* Inverse for float32 scales: bf16(float(value(q) * s)), one float product
 * rounded to nearest even in bf16.  NaN codes, and NaN products (a zero code
 * times an infinite scale), give a quiet NaN with the code's sign (the scale
 * is never negative; IEEE leaves the sign of such a NaN open). */
void eo_dequant_row_f32scale(const uint8_t* q, const float* scales, int32_t H, uint16_t* out)
{
    for (int32_t c = 0; c < H; ++c) {
        uint8_t b = q[c];
        if ((b & 0x7F) == 0x7F) {
            out[c] = (uint16_t)((b & 0x80 ? 0x8000 : 0) | 0x7FC0);
            continue;
        }
        float v = (float)eo_e4m3_value(b & 0x7F);
        if (b & 0x80)
            v = -v;
        float p = v * scales[c / 128];
        if (isnan(p))
            out[c] = (uint16_t)((b & 0x80 ? 0x8000 : 0) | 0x7FC0);
        else
            out[c] = eo_f32_to_bf16(p);
    }
}
