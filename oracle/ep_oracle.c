/*
 * ep_oracle.c -- CPU oracle for MoE expert-parallel route / dispatch / combine.
 *
 * TEST INFRASTRUCTURE ONLY: loaded by the tests, the smoke check and the
 * benchmark's CPU-baseline leg, never by the product library.  Plain C,
 * single-threaded, no blocking, no fusion; floating point in double.
 * Built with -ffp-contract=off so every expression rounds as written.
 * The page citations are spelled out in ep_oracle.h.
 */
#include "ep_oracle.h"

#include <math.h>
#include <stdlib.h>
#include <string.h>

/* ------------------------------------------------------------------------ */
/* bf16 format: 1 sign bit, 8 exponent bits (bias 127), 7 fraction bits.     */
/* ------------------------------------------------------------------------ */

double ep_oracle_bf16_to_double(uint16_t b)
{
    int sign = (b >> 15) & 1;
    int expo = (b >> 7) & 0xFF;
    int frac = b & 0x7F;
    double mag;
    if (expo == 0xFF) {
        mag = frac ? NAN : INFINITY;
    } else if (expo == 0) {
        mag = ldexp((double)frac, -126 - 7);            /* subnormal: 0.frac * 2^-126 */
    } else {
        mag = ldexp(128.0 + (double)frac, expo - 127 - 7); /* 1.frac * 2^(expo-127) */
    }
    return sign ? -mag : mag;
}

/* Round a double to the nearest bf16, ties to even, in one step (no detour
 * through float, which could round twice).  The quantum (spacing of bf16
 * values) next to |v| is 2^(e-8) for |v| in [2^(e-1), 2^e), never below the
 * subnormal spacing 2^-133.  Overflow goes to infinity; NaN stays NaN (quiet,
 * sign kept). */
uint16_t ep_oracle_double_to_bf16(double v)
{
    uint16_t sign = signbit(v) ? 0x8000u : 0u;
    if (isnan(v)) return (uint16_t)(sign | 0x7FC0u);
    double a = fabs(v);
    if (isinf(a)) return (uint16_t)(sign | 0x7F80u);
    if (a == 0.0) return sign;

    int e;
    (void)frexp(a, &e);                 /* a = m * 2^e, m in [0.5, 1) */
    int qexp = e - 8;
    if (qexp < -133) qexp = -133;
    double q = nearbyint(ldexp(a, -qexp)); /* RNE under the default rounding mode */
    double r = ldexp(q, qexp);             /* exact: q has at most 9 bits */

    if (r >= ldexp(1.0, 128)) return (uint16_t)(sign | 0x7F80u);

    /* r is now a bf16 value; encode it from the format's definition. */
    if (r < ldexp(1.0, -126)) {                       /* subnormal (or zero) */
        int frac = (int)ldexp(r, 133);
        return (uint16_t)(sign | (uint16_t)frac);
    }
    int er;
    double mr = frexp(r, &er);                        /* r = mr * 2^er, mr in [0.5,1) */
    int expo = er - 1 + 127;                          /* r = 1.f * 2^(er-1) */
    int frac = (int)ldexp(mr, 8) - 128;               /* 8 significant bits */
    return (uint16_t)(sign | (uint16_t)(expo << 7) | (uint16_t)frac);
}

/* ------------------------------------------------------------------------ */
/* Route: top-k selection + softmax gating.                                  */
/* HyperParallel-MoE sec. 2.2: the router picks a small subset of experts per */
/* token by top-k routing and their outputs are weighted by routing scores.  */
/* ------------------------------------------------------------------------ */

/* "a ranks before b": larger logit first, equal logits -> lower index. */
static int ranks_before(float la, int a, float lb, int b)
{
    if (la > lb) return 1;
    if (la < lb) return 0;
    return a < b;
}

int ep_oracle_route_topk(const float* logits, int64_t T, int32_t E, int32_t k,
                         int32_t normalize, int32_t* topk_idx, float* topk_w)
{
    if (!logits || !topk_idx || !topk_w || T < 0 || E < 1 || k < 1 || k > E)
        return -1;
    char* taken = (char*)malloc((size_t)E);
    double* ex = (double*)malloc(sizeof(double) * (size_t)k);
    if (!taken || !ex) { free(taken); free(ex); return -2; }

    for (int64_t t = 0; t < T; ++t) {
        const float* l = logits + t * (int64_t)E;
        int32_t* idx = topk_idx + t * (int64_t)k;
        float* w = topk_w + t * (int64_t)k;
        for (int32_t e = 0; e < E; ++e) {
            if (!isfinite(l[e])) { free(taken); free(ex); return -3; }
        }

        /* Selection: k passes, each picks the best expert not yet taken. */
        memset(taken, 0, (size_t)E);
        for (int32_t j = 0; j < k; ++j) {
            int best = -1;
            for (int32_t e = 0; e < E; ++e) {
                if (taken[e]) continue;
                if (best < 0 || ranks_before(l[e], e, l[best], best)) best = e;
            }
            taken[best] = 1;
            idx[j] = best;
        }

        /* Gating weights.  The first pick holds the largest logit m; shifting
         * every exponent by m leaves each ratio unchanged. */
        double m = (double)l[idx[0]];
        if (normalize) {
            double s = 0.0;
            for (int32_t j = 0; j < k; ++j) {
                ex[j] = exp((double)l[idx[j]] - m);
                s += ex[j];
            }
            for (int32_t j = 0; j < k; ++j) w[j] = (float)(ex[j] / s);
        } else {
            double z = 0.0;
            for (int32_t e = 0; e < E; ++e) z += exp((double)l[e] - m);
            for (int32_t j = 0; j < k; ++j)
                w[j] = (float)(exp((double)l[idx[j]] - m) / z);
        }
    }
    free(taken);
    free(ex);
    return 0;
}

/* ------------------------------------------------------------------------ */
/* Dispatch layout.                                                          */
/* UBEP sec. 2.3 / Fig. 2: per-expert token counts, then offset calculation  */
/* and a contiguous reordering; sec. 3.2: prefix sums give each expert's     */
/* offset.  StrataCL appendix (Hierarchical Workload Partitioning): the      */
/* token-placement metadata is destination expert, per-expert counts,        */
/* prefix-sum offsets and token-local offsets.  Written here as a stable     */
/* counting sort of the flattened slots s = t*k + j by expert.               */
/* ------------------------------------------------------------------------ */

int ep_oracle_dispatch_layout(const int32_t* topk_idx, int64_t T, int32_t k,
                              int32_t E, int32_t R, int32_t* expert_counts,
                              int32_t* expert_offsets, int32_t* rank_counts,
                              int32_t* rank_offsets, int32_t* pos,
                              int32_t* slot_src)
{
    if (!topk_idx || !expert_counts || !expert_offsets || !rank_counts ||
        !rank_offsets || !pos || T < 0 || k < 1 || E < 1 || R < 1 || E % R != 0)
        return -1;
    const int64_t S = T * (int64_t)k;
    if (S >= ((int64_t)1 << 30)) return -1;
    const int32_t L = E / R;                    /* experts per virtual rank */

    /* 1. per-expert counts */
    for (int32_t e = 0; e < E; ++e) expert_counts[e] = 0;
    for (int64_t s = 0; s < S; ++s) {
        int32_t e = topk_idx[s];
        if (e < 0 || e >= E) return -4;
        expert_counts[e] += 1;
    }
    /* 2. exclusive prefix sum -> per-expert offsets */
    expert_offsets[0] = 0;
    for (int32_t e = 0; e < E; ++e)
        expert_offsets[e + 1] = expert_offsets[e] + expert_counts[e];
    /* 3. rank r owns experts [r*L, r*L + L): its segment of the send buffer */
    for (int32_t r = 0; r < R; ++r) {
        rank_offsets[r] = expert_offsets[r * L];
        rank_counts[r] = 0;
        for (int32_t i = 0; i < L; ++i) rank_counts[r] += expert_counts[r * L + i];
    }
    rank_offsets[R] = expert_offsets[E];
    /* 4. token-local offsets: walk the slots in order, each takes the next free
     *    place of its expert (this is what makes the order stable) */
    int32_t* cursor = (int32_t*)malloc(sizeof(int32_t) * (size_t)E);
    if (!cursor) return -2;
    for (int32_t e = 0; e < E; ++e) cursor[e] = expert_offsets[e];
    for (int64_t s = 0; s < S; ++s) {
        int32_t e = topk_idx[s];
        pos[s] = cursor[e]++;
        if (slot_src) slot_src[pos[s]] = (int32_t)s;
    }
    free(cursor);
    return 0;
}

/* ------------------------------------------------------------------------ */
/* Dispatch: UBEP sec. 2.1 / 2.3 -- each token's activation goes to every    */
/* expert it picked; a token may be sent to several experts.                 */
/* ------------------------------------------------------------------------ */

int ep_oracle_dispatch(const uint16_t* x, int64_t T, int32_t H, int32_t k,
                       const int32_t* pos, uint16_t* send)
{
    if (!x || !pos || !send || T < 0 || H < 1 || k < 1) return -1;
    const int64_t S = T * (int64_t)k;
    for (int64_t t = 0; t < T; ++t) {
        for (int32_t j = 0; j < k; ++j) {
            int64_t p = pos[t * k + j];
            if (p < 0 || p >= S) return -4;
            memcpy(send + p * (int64_t)H, x + t * (int64_t)H, sizeof(uint16_t) * (size_t)H);
        }
    }
    return 0;
}

/* ------------------------------------------------------------------------ */
/* Combine: HyperParallel-MoE sec. 4.1 -- the top-k expert contributions are */
/* accumulated according to the routing scores; RailWave "System Design" --  */
/* combine uses the dispatch metadata to put outputs back at their original  */
/* token positions.                                                          */
/*                                                                           */
/* The value the library computes (the contract): fp32 accumulation in the  */
/* fixed top-k order j = 0..k-1.  acc = w0 * y0 as one fp32 product (one    */
/* rounding), then acc = fmaf(wj, yj, acc) for j = 1..k-1 (one rounding     */
/* each), then one round-to-nearest-even to bf16.  This file is built with  */
/* -ffp-contract=off, so the product of pick 0 is never fused into the next */
/* step, and fmaf is C99's correctly rounded fused multiply-add.            */
/*                                                                           */
/* The exact value (the accuracy reference): the same sum in double, where  */
/* every product w*y of an fp32 weight and a bf16 value is exact, rounded   */
/* once to bf16.                                                            */
/* ------------------------------------------------------------------------ */

/* A bf16 pattern is the upper half of the binary32 pattern of the same
 * value, so widening is exact. */
static float bf16_to_float(uint16_t b)
{
    uint32_t u = (uint32_t)b << 16;
    float f;
    memcpy(&f, &u, sizeof f);
    return f;
}

static void combine_one(const uint16_t* y, const int32_t* pos, const float* topk_w,
                        int64_t t, int32_t H, int32_t k, uint16_t* out_row)
{
    const int32_t* p = pos + t * (int64_t)k;
    const float* w = topk_w + t * (int64_t)k;
    for (int32_t h = 0; h < H; ++h) {
        float acc = w[0] * bf16_to_float(y[(int64_t)p[0] * H + h]);
        for (int32_t j = 1; j < k; ++j)
            acc = fmaf(w[j], bf16_to_float(y[(int64_t)p[j] * H + h]), acc);
        /* float -> double is exact, so this is one rounding to bf16. */
        out_row[h] = ep_oracle_double_to_bf16((double)acc);
    }
}

static void combine_exact_one(const uint16_t* y, const int32_t* pos, const float* topk_w,
                              int64_t t, int32_t H, int32_t k, uint16_t* out_row)
{
    const int32_t* p = pos + t * (int64_t)k;
    const float* w = topk_w + t * (int64_t)k;
    for (int32_t h = 0; h < H; ++h) {
        double acc = (double)w[0] * ep_oracle_bf16_to_double(y[(int64_t)p[0] * H + h]);
        for (int32_t j = 1; j < k; ++j)
            acc = acc + (double)w[j] * ep_oracle_bf16_to_double(y[(int64_t)p[j] * H + h]);
        out_row[h] = ep_oracle_double_to_bf16(acc);
    }
}

static int check_pos(const int32_t* pos, int64_t T, int32_t k)
{
    const int64_t S = T * (int64_t)k;
    for (int64_t s = 0; s < S; ++s)
        if (pos[s] < 0 || pos[s] >= S) return -4;
    return 0;
}

int ep_oracle_combine(const uint16_t* y, const int32_t* pos, const float* topk_w,
                      int64_t T, int32_t H, int32_t k, uint16_t* out)
{
    if (!y || !pos || !topk_w || !out || T < 0 || H < 1 || k < 1) return -1;
    if (check_pos(pos, T, k)) return -4;
    for (int64_t t = 0; t < T; ++t)
        combine_one(y, pos, topk_w, t, H, k, out + t * (int64_t)H);
    return 0;
}

int ep_oracle_combine_exact(const uint16_t* y, const int32_t* pos, const float* topk_w,
                            int64_t T, int32_t H, int32_t k, uint16_t* out)
{
    if (!y || !pos || !topk_w || !out || T < 0 || H < 1 || k < 1) return -1;
    if (check_pos(pos, T, k)) return -4;
    for (int64_t t = 0; t < T; ++t)
        combine_exact_one(y, pos, topk_w, t, H, k, out + t * (int64_t)H);
    return 0;
}

int ep_oracle_combine_tokens(const uint16_t* y, const int32_t* pos,
                             const float* topk_w, int64_t T, int32_t H, int32_t k,
                             const int64_t* tokens, int64_t n_tokens,
                             uint16_t* out_rows)
{
    if (!y || !pos || !topk_w || !tokens || !out_rows || T < 0 || H < 1 || k < 1 ||
        n_tokens < 0)
        return -1;
    if (check_pos(pos, T, k)) return -4;
    for (int64_t i = 0; i < n_tokens; ++i) {
        if (tokens[i] < 0 || tokens[i] >= T) return -1;
        combine_one(y, pos, topk_w, tokens[i], H, k, out_rows + i * (int64_t)H);
    }
    return 0;
}

/* ------------------------------------------------------------------------ */
/* Flag-in-payload trailer.  UBEP sec. 3.4 / Fig. 6 (Token-Flag Fusion): the */
/* readiness flag travels inside the data block, so seeing the flag proves   */
/* the block arrived.  Read here as one 16-byte trailer after each row:      */
/* the call's 64-bit epoch, then the slot's source index, then zero.         */
/* ------------------------------------------------------------------------ */

int ep_oracle_fused_trailer(uint64_t epoch, const int32_t* slot_src, int64_t slot,
                            uint8_t trailer[16])
{
    if (!slot_src || !trailer || slot < 0) return -1;
    uint32_t src = (uint32_t)slot_src[slot];
    for (int i = 0; i < 8; ++i) trailer[i] = (uint8_t)(epoch >> (8 * i));
    for (int i = 0; i < 4; ++i) trailer[8 + i] = (uint8_t)(src >> (8 * i));
    for (int i = 0; i < 4; ++i) trailer[12 + i] = 0;
    return 0;
}

/* ------------------------------------------------------------------------ */
/* Backward pass [HPMOE sec. 2.2, Fig. 2(b)]: the backward Dispatch is the    */
/* gradient of the forward Combine, the backward Combine returns the          */
/* gradient of the input activations.                                         */
/* ------------------------------------------------------------------------ */

int ep_oracle_combine_grad(const uint16_t* grad_out, const uint16_t* y,
                           const int32_t* pos, const float* topk_w,
                           int64_t T, int32_t H, int32_t k,
                           uint16_t* grad_y, double* grad_w)
{
    if (!grad_out || !y || !pos || !topk_w || !grad_y || !grad_w || T < 0 || H < 1 || k < 1)
        return -1;
    if (check_pos(pos, T, k) != 0) return -4;
    for (int64_t t = 0; t < T; ++t) {
        const uint16_t* g = grad_out + t * (int64_t)H;
        for (int32_t j = 0; j < k; ++j) {
            const int64_t p = pos[t * k + j];
            const double w = (double)topk_w[t * k + j];
            const uint16_t* yr = y + p * (int64_t)H;
            uint16_t* gy = grad_y + p * (int64_t)H;
            double dot = 0.0;
            for (int32_t h = 0; h < H; ++h) {
                const double gh = ep_oracle_bf16_to_double(g[h]);
                /* d out[t][h] / d y[p][h] = w: the exact product (24 x 8
                 * significant bits fits a double), rounded once to bf16. */
                gy[h] = ep_oracle_double_to_bf16(w * gh);
                /* d out[t][h] / d w = y[p][h]; summed over h against g. */
                dot = dot + gh * ep_oracle_bf16_to_double(yr[h]);
            }
            grad_w[t * k + j] = dot;
        }
    }
    return 0;
}

int ep_oracle_dispatch_grad(const uint16_t* grad_send, const int32_t* pos,
                            int64_t T, int32_t H, int32_t k, uint16_t* grad_x)
{
    if (!grad_send || !pos || !grad_x || T < 0 || H < 1 || k < 1) return -1;
    if (check_pos(pos, T, k) != 0) return -4;
    for (int64_t t = 0; t < T; ++t) {
        for (int32_t h = 0; h < H; ++h) {
            /* x[t] was copied to every row pos[t][j]: its gradient is the sum
             * of those rows' gradients, accumulated in fp32 in pick order
             * (one rounding per addition), then rounded once to bf16. */
            float acc = bf16_to_float(grad_send[(int64_t)pos[t * k] * H + h]);
            for (int32_t j = 1; j < k; ++j)
                acc = acc + bf16_to_float(grad_send[(int64_t)pos[t * k + j] * H + h]);
            grad_x[t * (int64_t)H + h] = ep_oracle_double_to_bf16((double)acc);
        }
    }
    return 0;
}

int ep_oracle_dispatch_grad_exact(const uint16_t* grad_send, const int32_t* pos,
                                  int64_t T, int32_t H, int32_t k, uint16_t* grad_x)
{
    if (!grad_send || !pos || !grad_x || T < 0 || H < 1 || k < 1) return -1;
    if (check_pos(pos, T, k) != 0) return -4;
    for (int64_t t = 0; t < T; ++t) {
        for (int32_t h = 0; h < H; ++h) {
            /* The same sum in double, rounded once to bf16: the accuracy
             * reference for the fp32 sum above. */
            double acc = 0.0;
            for (int32_t j = 0; j < k; ++j) {
                const int64_t p = pos[t * k + j];
                acc = acc + ep_oracle_bf16_to_double(grad_send[p * (int64_t)H + h]);
            }
            grad_x[t * (int64_t)H + h] = ep_oracle_double_to_bf16(acc);
        }
    }
    return 0;
}

/* ------------------------------------------------------------------------ */
/* Skew-balanced work partition.                                             */
/* ------------------------------------------------------------------------ */

int ep_oracle_slices(const int32_t* expert_offsets, int32_t E, int32_t P,
                     int64_t* start, int32_t* expert, int64_t* offset)
{
    if (!expert_offsets || !start || !expert || !offset || E < 1 || P < 1) return -1;
    const int64_t S = expert_offsets[E];
    for (int32_t e = 0; e < E; ++e)
        if (expert_offsets[e + 1] < expert_offsets[e]) return -2;
    for (int32_t p = 0; p <= P; ++p) {
        /* [UBEP sec. 3.3, token-level load partition] equal contiguous slices:
         * slice p is [floor(p*S/P), floor((p+1)*S/P)), sizes differ by <= 1. */
        start[p] = (p * S) / P;
        if (p == P) break;
        /* the expert whose cumulative range [offsets[e], offsets[e+1])
         * covers the slice start, and the start's offset inside it; a start
         * at S (an empty last slice) maps to expert E, offset 0 */
        expert[p] = E;
        offset[p] = 0;
        for (int32_t e = 0; e < E; ++e) {
            if (expert_offsets[e] <= start[p] && start[p] < expert_offsets[e + 1]) {
                expert[p] = e;
                offset[p] = start[p] - expert_offsets[e];
                break;
            }
        }
    }
    return 0;
}

int ep_oracle_lpt(const double* cost, const int32_t* peer, int32_t U,
                  const int32_t* cap_of_peer, int32_t npeer, int32_t C,
                  int32_t* core, int32_t* stripe, double* load)
{
    if (!cost || !peer || !cap_of_peer || !core || !stripe || !load || U < 0 || C < 1 ||
        npeer < 1)
        return -1;
    for (int32_t p = 0; p < npeer; ++p)
        if (cap_of_peer[p] < 1) return -2;
    for (int32_t j = 0; j < U; ++j)
        if (peer[j] < 0 || peer[j] >= npeer) return -3;
    /* [StrataCL sec. 6.2, App. B] LPT-style list scheduling: units in order
     * of decreasing estimated cost (equal costs: lower index first), each to
     * the least-loaded core (ties: lower index) whose next stripe still has
     * room for the unit's peer under the fan-out cap.  A core issues at most
     * one unit per stripe, so its next stripe is its count of stripes so far.
     * When no core has room, the least-loaded core skips stripes (idle) until
     * its next stripe has room. */
    int32_t* order = (int32_t*)malloc(sizeof(int32_t) * (size_t)(U > 0 ? U : 1));
    int32_t* next = (int32_t*)calloc((size_t)C, sizeof(int32_t));
    /* fan-out counts per (stripe, peer).  A core's next stripe grows by one
     * per unit it takes plus one per stripe it skips; a skipped stripe is full
     * for some peer, and there are at most U such stripes, so 2U + 2 rows
     * bound the table. */
    const int64_t maxk = 2 * (int64_t)U + 2;
    int32_t* fan = (int32_t*)calloc((size_t)(maxk * npeer), sizeof(int32_t));
    if (!order || !next || !fan) { free(order); free(next); free(fan); return -4; }
    for (int32_t j = 0; j < U; ++j) order[j] = j;
    for (int32_t a = 1; a < U; ++a) {          /* insertion sort: stable */
        const int32_t v = order[a];
        int32_t b = a - 1;
        while (b >= 0 && cost[order[b]] < cost[v]) { order[b + 1] = order[b]; --b; }
        order[b + 1] = v;
    }
    for (int32_t c = 0; c < C; ++c) load[c] = 0.0;
    int rc = 0;
    for (int32_t i = 0; i < U; ++i) {
        const int32_t j = order[i];
        const int32_t p = peer[j];
        int32_t best = -1;
        for (int32_t c = 0; c < C; ++c) {
            if (fan[(int64_t)next[c] * npeer + p] >= cap_of_peer[p]) continue;
            if (best < 0 || load[c] < load[best]) best = c;
        }
        if (best < 0) {
            for (int32_t c = 0; c < C; ++c)
                if (best < 0 || load[c] < load[best]) best = c;
            while (next[best] < maxk && fan[(int64_t)next[best] * npeer + p] >= cap_of_peer[p])
                ++next[best];
        }
        if (next[best] >= maxk) { rc = -5; break; }
        core[j] = best;
        stripe[j] = next[best];
        fan[(int64_t)next[best] * npeer + p] += 1;
        next[best] += 1;
        load[best] += cost[j];
    }
    free(order);
    free(next);
    free(fan);
    return rc;
}

/* ------------------------------------------------------------------------ */
/* Rank-level token coalescing: RailWave sec. 3.1-3.2 -- transfer records   */
/* per destination keep the backend's token coalescing; a record may carry  */
/* several destinations of one token.  One record per (token, rank).        */
/* ------------------------------------------------------------------------ */

int64_t ep_oracle_rank_coalesce(const int32_t* topk_idx, int64_t T, int32_t k, int32_t E,
                                int32_t R, int32_t* rank_counts, int32_t* rank_offsets,
                                int32_t* row_of_pick, int32_t* send_pos, int32_t* row_src,
                                uint64_t* row_experts)
{
    if (!topk_idx || !rank_counts || !rank_offsets || !row_of_pick || !send_pos ||
        !row_src || !row_experts || T < 0 || k < 1 || E < 1 || R < 1 || E % R != 0)
        return -1;
    const int32_t L = E / R;
    if (L > 64) return -2;
    const int64_t S = T * (int64_t)k;
    for (int64_t s = 0; s < S; ++s)
        if (topk_idx[s] < 0 || topk_idx[s] >= E) return -4;

    /* first[s]: pick s = t*k + j is the token's first pick of its rank */
    unsigned char* first = (unsigned char*)malloc((size_t)(S > 0 ? S : 1));
    if (!first) return -5;
    for (int64_t t = 0; t < T; ++t)
        for (int32_t j = 0; j < k; ++j) {
            const int32_t r = topk_idx[t * k + j] / L;
            int f = 1;
            for (int32_t i = 0; i < j; ++i)
                if (topk_idx[t * k + i] / L == r) f = 0;
            first[t * k + j] = (unsigned char)f;
        }

    /* records per rank, and where each rank's records start */
    for (int32_t r = 0; r < R; ++r) rank_counts[r] = 0;
    for (int64_t s = 0; s < S; ++s)
        if (first[s]) rank_counts[topk_idx[s] / L] += 1;
    int64_t run = 0;
    for (int32_t r = 0; r < R; ++r) {
        rank_offsets[r] = (int32_t)run;
        run += rank_counts[r];
    }
    rank_offsets[R] = (int32_t)run;

    /* rows in token order inside each rank */
    int32_t* cursor = (int32_t*)malloc(sizeof(int32_t) * (size_t)R);
    if (!cursor) { free(first); return -5; }
    for (int32_t r = 0; r < R; ++r) cursor[r] = rank_offsets[r];
    for (int64_t t = 0; t < T; ++t) {
        for (int32_t j = 0; j < k; ++j) {
            const int64_t s = t * k + j;
            const int32_t r = topk_idx[s] / L;
            if (first[s]) {
                const int32_t row = cursor[r]++;
                row_src[row] = (int32_t)t;
                row_experts[row] = 0;
                row_of_pick[s] = row;
                send_pos[s] = row;
            } else {
                int32_t j0 = 0;
                while (topk_idx[t * k + j0] / L != r) ++j0;
                row_of_pick[s] = row_of_pick[t * k + j0];
                send_pos[s] = -1;
            }
            row_experts[row_of_pick[s]] |= (uint64_t)1 << (topk_idx[s] % L);
        }
    }
    free(cursor);
    free(first);
    return run;
}

/* Receiver-side expansion of coalesced records: RailWave sec. 3.1-3.2 and   */
/* StrataCL's level-2 expert windows -- a stable counting sort of the        */
/* (record, local expert) pairs by expert.                                    */
int ep_oracle_expand_records(const uint64_t* masks, int64_t C, int32_t L, int32_t* expert_counts,
                             int32_t* expert_offsets, int32_t* pos)
{
    if (!masks || !expert_counts || !expert_offsets || !pos || C < 0 || L < 1 || L > 64)
        return -1;
    for (int32_t i = 0; i < L; ++i) expert_counts[i] = 0;
    for (int64_t c = 0; c < C; ++c) {
        if (L < 64 && (masks[c] >> L) != 0) return -2;       /* a bit past the last expert */
        for (int32_t i = 0; i < L; ++i)
            if ((masks[c] >> i) & 1u) expert_counts[i] += 1;
    }
    int64_t run = 0;
    for (int32_t i = 0; i < L; ++i) {
        expert_offsets[i] = (int32_t)run;
        run += expert_counts[i];
    }
    expert_offsets[L] = (int32_t)run;
    for (int32_t i = 0; i < L; ++i) {
        int64_t next = expert_offsets[i];
        for (int64_t c = 0; c < C; ++c)
            pos[c * L + i] = ((masks[c] >> i) & 1u) ? (int32_t)next++ : -1;
    }
    return 0;
}

/* Cyclic exchange waves: RailWave sec. 3.2, eq. (10). */
int ep_oracle_exchange_waves(int32_t N, int32_t* peer)
{
    if (N < 1 || !peer) return -1;
    for (int32_t k = 1; k < N; ++k)
        for (int32_t s = 0; s < N; ++s)
            peer[(int64_t)(k - 1) * N + s] = (s + k) % N;
    return 0;
}

/* Incast degree of a wave: RailWave App. A.6, Table 8 ("peak incast"). */
int32_t ep_oracle_incast_degree(const int32_t* dst, int32_t N)
{
    if (N < 1 || !dst) return -1;
    int32_t best = 0;
    for (int32_t d = 0; d < N; ++d) {
        int32_t n = 0;
        for (int32_t s = 0; s < N; ++s)
            if (dst[s] == d && s != d) ++n;
        if (n > best) best = n;
    }
    return best;
}
