/*
 * moe_oracle.c -- plain, slow CPU oracle for the MoE layer forward pass.
 *
 * TEST INFRASTRUCTURE ONLY.  Nothing in the product path may link, load or
 * call this file; only the test suite, the smoke check and the CPU-baseline
 * leg of the benchmark do.  It shares no code, header, table or helper with
 * the GPU library: it is written from the page definitions alone.
 *
 * Arithmetic: every accumulation is in IEEE double.  Values are rounded to
 * fp32 or bf16 (round-to-nearest-even, computed from the exact double) only
 * at the points where the method stores a tensor:
 *   logits            -> fp32
 *   gate weights      -> fp32
 *   SwiGLU hidden h   -> bf16
 *   expert output     -> bf16
 *   layer output y    -> bf16
 *
 * Sources (page title, section):
 *   [G]  "Mixture-of-Experts (MoE) Architecture and Expert Parallelism",
 *        section 2 "The Gating Network Formulation": H(x) = x W_g + eps,
 *        G(x) = Softmax(KeepTopK(H(x), K)), KeepTopK keeps the K largest
 *        coordinates and sets the rest to -inf, y = sum_{i in TopK} G_i Expert_i(x).
 *   [N]  "EP Math -- Expert Parallelism (MoE)", "Notation": T tokens per
 *        device, d hidden size, T*k assignments per device.
 *   [DA] same page, "The dispatch all-to-all": T*k*d*2 bytes produced,
 *        (D-1)/D of it leaves the device.
 *   [CA] same page, "The combine all-to-all": the exact reverse of dispatch,
 *        weighted by the gate values and summed at the token's home device.
 *   [CF] same page, "Capacity factor": C = f * tokens * k / E, rounded up;
 *        buffer [E, C, d]; under-full experts padded up to C.
 *   [TD] same page, "Token drop": assignments beyond C are dropped and the
 *        token passes as if that expert's output were zero.
 *   [PL] same page, "Placing experts across devices": E/D whole experts per
 *        device, E divisible by D.
 *   [M]  "MoE Expert Parallelism Sizing: Traffic, Capacity, Fabric",
 *        "Memory residency for the same shape": gated three-matrix expert
 *        (3*d*H parameters); "Capacity semantics decide what crosses the
 *        wire": dropping happens before the exchange; "First-order dispatch
 *        and combine bytes": one input chunk per destination rank.
 *   [DP] same page, "Capacity semantics decide what crosses the wire", and
 *        its question on the capacity factor: with a capacity factor set,
 *        the tokens beyond an expert's capacity are dropped by their
 *        selected (gate) probability, the default strategy drops nothing.
 *   [MC] same page, the DeepSpeed paragraph: C raised to a floor,
 *        min_capacity, whatever the capacity factor gives.
 *   [F8] same page, "What the bounds omit": FP8 rows on dispatch, bf16 on
 *        combine; per-row scales added to the traffic.
 *   [GL] same page, the traffic bounds: DeepSeek-V3 dispatches each token
 *        to at most 4 nodes, which Megatron exposes as group-limited
 *        routing.
 *   [SE] same page, the token-assignment worksheet: the shared expert is
 *        replicated on every EP rank (compute and memory, no dispatch
 *        traffic) in Megatron, or routed as a ninth expert in DeepSeek's
 *        decode deployment.
 *
 * Readings taken where the pages are silent (each also listed in the design
 * notes): eps = 0 at inference; an optional per-expert logit bias b is added
 * to H and enters both selection and softmax; ties in KeepTopK go to the
 * lower expert index; the kept experts are reported in descending-logit
 * order; capacity uses the per-device token count T, computed as
 * ceil(cf*T*k/E) in double, raised to a minimum capacity when one is given
 * [MC]; overflow is dropped in token order (the first C assignments of an
 * expert, by token index, are kept) under drop policy 0, or by gate
 * probability under drop policy 1 [DP]: the C assignments with the largest
 * gate value G stay, equal G going to the lower token index, and the kept
 * rows keep token order inside the expert's block; FP8 dispatch [F8] uses
 * the OCP E4M3 format (bias 7, max 448, no infinities) with one fp32 scale
 * per row, s = amax/448 computed in fp32 (s = 1 for an all-zero row), each
 * element encoded as E4M3(x/s) with x/s computed in fp32, rounded to the
 * nearest E4M3 value (ties to even), saturated at +-448, sign kept (so -0
 * and tiny negatives give 0x80); the expert sees code value * s, and the
 * combine stays bf16; group-limited routing [GL] splits the E experts into
 * G equal contiguous groups, scores each group by its largest logit for
 * the token, keeps the M best groups (ties to the lower group index) and
 * runs KeepTopK over their experts only; the shared expert [SE] follows
 * the replicated convention: a SwiGLU of every token, bf16 output, added
 * with weight 1 in the combine; gates are not
 * renormalised after a drop; a routing entry outside [0, E) or repeating
 * an expert already listed for its token is invalid (counted, dropped),
 * since KeepTopK yields k distinct experts; the expert is SwiGLU, W2 (SiLU(W1 x) * (W3 x))
 * with no biases; placement is contiguous: rank r owns experts
 * [r*E/D, (r+1)*E/D).
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>
#ifdef _OPENMP
#include <omp.h>
#endif

/* ------------------------------------------------------------------ */
/* Number formats.                                                     */
/* ------------------------------------------------------------------ */

/* bf16 is the upper 16 bits of an IEEE binary32. */
static double bf16_value(uint16_t b)
{
    uint32_t u = (uint32_t)b << 16;
    float f;
    memcpy(&f, &u, sizeof f);
    return (double)f;
}

/* Round a finite double to the nearest bf16 (ties to even) in one step.
 * bf16 keeps 8 significant bits and fp32's exponent range, so its spacing
 * near |v| in [2^e, 2^(e+1)) is 2^(e-7), and 2^-133 below 2^-126. */
uint16_t oracle_bf16_from_double(double v)
{
    uint16_t sign = signbit(v) ? 0x8000u : 0u;
    if (isnan(v))
        return 0x7FC0u;
    if (v == 0.0)
        return sign;
    int ex;
    frexp(v, &ex); /* |v| = m * 2^ex with m in [0.5, 1) */
    int q = ex - 8; /* spacing exponent for 8 significant bits */
    if (q < -133)
        q = -133;
    double r = ldexp(nearbyint(ldexp(v, -q)), q); /* exact scaling, RNE */
    if (isinf(r) || fabs(r) >= ldexp(1.0, 128))
        return (uint16_t)(sign | 0x7F80u);
    float f = (float)r; /* exact: r has at most 8 significant bits */
    uint32_t u;
    memcpy(&u, &f, sizeof u);
    return (uint16_t)(u >> 16);
}

/* ------------------------------------------------------------------ */
/* Step 1: router logits  H = x W_g (+ b),  eps = 0.        [G]        */
/* x [T, d] bf16, w_gate [d, E] bf16 (d_model x E as on the page),     */
/* bias [E] fp32 or NULL, logits [T, E] fp32.                          */
/* ------------------------------------------------------------------ */
void oracle_logits(int T, int d, int E, const uint16_t *x, const uint16_t *w_gate,
                   const float *bias, float *logits)
{
#pragma omp parallel for schedule(static)
    for (int t = 0; t < T; ++t) {
        for (int e = 0; e < E; ++e) {
            double acc = 0.0;
            for (int j = 0; j < d; ++j)
                acc += bf16_value(x[(size_t)t * d + j]) * bf16_value(w_gate[(size_t)j * E + e]);
            if (bias)
                acc += (double)bias[e];
            logits[(size_t)t * E + e] = (float)acc;
        }
    }
}

/* ------------------------------------------------------------------ */
/* Step 2: G = Softmax(KeepTopK(H, k)).                  [G][GL]       */
/* Group limit (G groups of E/G contiguous experts, at most M groups   */
/* per token; G <= 1 or M >= G means no limit): group g's score is the */
/* largest logit of its experts; group rank(g) = #{g' : s_g' > s_g, or */
/* s_g' == s_g and g' < g}; the experts of groups with rank < M are    */
/* allowed, the others act as -inf.                                     */
/* KeepTopK by rank among allowed experts: rank(e) = #{allowed e' :    */
/* h_e' > h_e, or h_e' == h_e and e' < e}.  Expert e is kept iff       */
/* rank(e) < k; it is written to output position rank(e).  The softmax */
/* over the kept logits equals the softmax over the KeepTopK vector,   */
/* whose other entries are -inf and contribute exp(-inf) = 0.          */
/* gap[t] = h_(k) - h_(k+1) among the allowed experts (+inf when all   */
/* are kept), and under a group limit also at most s_(M) - s_(M+1):    */
/* the distance to the nearest change of the selection.                */
/* Returns 0, or -1 (nothing written) for a shape beyond the per-token  */
/* scratch arrays (E > 4096, G > 1024) or without a valid selection    */
/* (k outside [1, E]; under a group limit E % G != 0, M < 1, or fewer  */
/* than k experts in M groups).                                        */
/* ------------------------------------------------------------------ */
#define TOPK_MAX_E 4096
#define TOPK_MAX_G 1024
int oracle_topk_grouped(int T, int E, int k, int G, int M, const float *logits,
                        int32_t *topk_idx, float *topk_w, double *gap)
{
    if (E < 1 || E > TOPK_MAX_E || G > TOPK_MAX_G || k < 1 || k > E)
        return -1;
    const int limited = G > 1 && M < G;
    if (limited && (E % G != 0 || M < 1 || (long)M * (E / G) < k))
        return -1;
    const int per = limited ? E / G : E;
#pragma omp parallel for schedule(static)
    for (int t = 0; t < T; ++t) {
        const float *h = logits + (size_t)t * E;
        double first_rejected = -INFINITY;
        int have_rejected = 0;
        double group_gap = INFINITY;
        /* allowed[e]: expert e's group is among the M best */
        char allowed[TOPK_MAX_E];
        for (int e = 0; e < E; ++e)
            allowed[e] = 1;
        if (limited) {
            float score[TOPK_MAX_G];
            for (int g = 0; g < G; ++g) {
                score[g] = h[g * per];
                for (int e = g * per + 1; e < (g + 1) * per; ++e)
                    if (h[e] > score[g])
                        score[g] = h[e];
            }
            double last_group = INFINITY, first_out = -INFINITY;
            for (int g = 0; g < G; ++g) {
                int grank = 0;
                for (int g2 = 0; g2 < G; ++g2)
                    if (score[g2] > score[g] || (score[g2] == score[g] && g2 < g))
                        ++grank;
                for (int e = g * per; e < (g + 1) * per; ++e)
                    allowed[e] = grank < M;
                if (grank == M - 1)
                    last_group = score[g];
                if (grank == M)
                    first_out = score[g];
            }
            group_gap = last_group - first_out;
        }
        for (int e = 0; e < E; ++e) {
            if (!allowed[e])
                continue;
            int rank = 0;
            for (int e2 = 0; e2 < E; ++e2)
                if (allowed[e2] && (h[e2] > h[e] || (h[e2] == h[e] && e2 < e)))
                    ++rank;
            if (rank < k) {
                topk_idx[(size_t)t * k + rank] = e;
            } else if (rank == k) {
                first_rejected = (double)h[e];
                have_rejected = 1;
            }
        }
        /* softmax over the kept logits, max-subtracted (the maximum is the
         * rank-0 entry); mathematically identical to the plain softmax */
        double hmax = (double)h[topk_idx[(size_t)t * k]];
        double denom = 0.0;
        for (int s = 0; s < k; ++s)
            denom += exp((double)h[topk_idx[(size_t)t * k + s]] - hmax);
        for (int s = 0; s < k; ++s)
            topk_w[(size_t)t * k + s] =
                (float)(exp((double)h[topk_idx[(size_t)t * k + s]] - hmax) / denom);
        if (gap) {
            double last_kept = (double)h[topk_idx[(size_t)t * k + k - 1]];
            double g_e = have_rejected ? last_kept - first_rejected : INFINITY;
            gap[t] = g_e < group_gap ? g_e : group_gap;
        }
    }
    return 0;
}

int oracle_topk(int T, int E, int k, const float *logits, int32_t *topk_idx,
                float *topk_w, double *gap)
{
    return oracle_topk_grouped(T, E, k, 1, 1, logits, topk_idx, topk_w, gap);
}

/* ------------------------------------------------------------------ */
/* Step 3: capacity.                                     [CF][MC]      */
/* C = ceil(cf * T * k / E) evaluated left to right in IEEE double,    */
/* then C = max(C, min_capacity).  cf = +inf means dropless; returns   */
/* -1 then (the minimum capacity does not apply).                      */
/* ------------------------------------------------------------------ */
int64_t oracle_capacity(int T, int k, int E, double cf, int min_capacity)
{
    if (isinf(cf))
        return -1;
    int64_t C = (int64_t)ceil(cf * (double)T * (double)k / (double)E);
    return C > min_capacity ? C : (int64_t)min_capacity;
}

/* Order of two assignments of one expert under drop policy 1: larger gate
 * value first, then lower token index (a token lists an expert once, so
 * the token decides every remaining tie).                       [DP]  */
static const float *g_cmp_w;
static int g_cmp_k;
static int by_gate_then_token(const void *pa, const void *pb)
{
    int32_t a = *(const int32_t *)pa, b = *(const int32_t *)pb;
    float ga = g_cmp_w[a], gb = g_cmp_w[b];
    if (ga != gb)
        return ga > gb ? -1 : 1;
    int32_t ta = a / g_cmp_k, tb = b / g_cmp_k;
    return (ta > tb) - (ta < tb);
}

/* ------------------------------------------------------------------ */
/* FP8 E4M3 (OCP) for the dispatch payload.                  [F8]      */
/* Code bits: s eeee mmm, exponent bias 7.  e = 0: subnormal m * 2^-9; */
/* e = 15, m = 7: NaN (never produced here); otherwise                 */
/* 2^(e-7) * (1 + m/8).  Largest finite value 448 (0x7E).              */
/* ------------------------------------------------------------------ */
double oracle_fp8_value(uint8_t code)
{
    int sgn = code >> 7, e = (code >> 3) & 15, m = code & 7;
    double v;
    if (e == 15 && m == 7)
        return NAN;
    if (e == 0)
        v = ldexp((double)m, -9);
    else
        v = ldexp(1.0 + m / 8.0, e - 7);
    return sgn ? -v : v;
}

/* Nearest E4M3 value to v (|v| saturated at 448), ties to the code with an
 * even mantissa, found by scanning every finite magnitude code. */
uint8_t oracle_fp8_from_float(float v)
{
    double a = fabs((double)v);
    if (a > 448.0)
        a = 448.0;
    int best = 0;
    double best_d = INFINITY;
    for (int c = 0; c <= 0x7E; ++c) {
        double dist = fabs(oracle_fp8_value((uint8_t)c) - a);
        if (dist < best_d || (dist == best_d && (c & 1) == 0 && (best & 1) == 1)) {
            best = c;
            best_d = dist;
        }
    }
    return (uint8_t)(best | (signbit(v) ? 0x80 : 0));
}

/* Per-row quantization of n bf16 rows [n, d]: scale s = amax / 448 (fp32),
 * code = E4M3(x / s) with the quotient in fp32.                      */
void oracle_fp8_quantize_rows(int n, int d, const uint16_t *x, uint8_t *codes, float *scales)
{
    for (int r = 0; r < n; ++r) {
        float amax = 0.0f;
        for (int i = 0; i < d; ++i) {
            float a = fabsf((float)bf16_value(x[(size_t)r * d + i]));
            if (a > amax)
                amax = a;
        }
        float sc = amax > 0.0f ? amax / 448.0f : 1.0f;
        scales[r] = sc;
        for (int i = 0; i < d; ++i) {
            float q = (float)bf16_value(x[(size_t)r * d + i]) / sc;
            codes[(size_t)r * d + i] = oracle_fp8_from_float(q);
        }
    }
}

/* Indices into the stats vector filled by oracle_dispatch. */
enum {
    ST_ASSIGNMENTS = 0, /* T*k                                          [N]  */
    ST_KEPT,            /* assignments that reach an expert                   */
    ST_DROPPED,         /* assignments - kept                            [TD] */
    ST_PADDED,          /* E*C - kept in capacity mode, else 0           [CF] */
    ST_CAPACITY,        /* C, or -1 when dropless                        [CF] */
    ST_SEND_ROWS,       /* rows of the send buffer: E*C, or T*k               */
    ST_DISPATCH_BYTES,  /* kept * d * 2: token vectors that travel       [DA] */
    ST_WIRE_BYTES,      /* send_rows * d * 2 in capacity mode (pads
                           included), kept*d*2 when dropless             [CF] */
    ST_REMOTE_BYTES,    /* kept rows bound for ranks != my_rank, *d*2    [DA] */
    ST_COMBINE_BYTES,   /* = dispatch bytes: combine reverses dispatch   [CA] */
    ST_MAX_COUNT,       /* max_e n_e                                          */
    ST_INVALID,         /* indices outside [0, E), or repeating an expert
                           already listed for the token: counted, dropped     */
    ST_COUNT
};

/* ------------------------------------------------------------------ */
/* Step 3/4: histogram, capacity, positions and the dispatch layout.   */
/*                                                   [N][CF][TD][PL][M] */
/* Positions: assignments are visited in ascending token order; the    */
/* position of (t, s) in expert e is the number of earlier tokens       */
/* routed to e (a token's k experts are distinct, so the slot order    */
/* inside one token never matters).  Drop policy 0: an assignment is   */
/* kept iff its position is below C.  Drop policy 1 [DP]: an expert    */
/* with more than C assignments keeps the C first in the order of      */
/* by_gate_then_token (topk_w holds G), and its kept assignments take  */
/* positions 0..C-1 in ascending token order.  The counts, and so the  */
/* offsets, bytes and per-rank rows, do not depend on the policy.      */
/* Layout: capacity mode gives expert e the rows                        */
/* [e*C, (e+1)*C) (pads left zero); dropless packs experts back to     */
/* back, offset_e = n_0 + ... + n_(e-1).  Experts are in ascending     */
/* order, so rank r's chunk -- the part the dispatch all-to-all sends  */
/* to rank r -- is rows [offset[r*E/D], offset[(r+1)*E/D]).            */
/* send_buf [send_rows, d] may be NULL (accounting only).              */
/* ------------------------------------------------------------------ */
int oracle_dispatch(int T, int d, int E, int k, int D, int my_rank, double cf,
                    int min_capacity, int drop_policy, int fp8, const uint16_t *x,
                    const int32_t *topk_idx, const float *topk_w, void *send_buf,
                    float *send_scale, int32_t *slot, int32_t *expert_count, int32_t *expert_kept,
                    int64_t *expert_offset, int64_t *rank_rows, int64_t *stats)
{
    if (D <= 0 || E % D != 0 || my_rank < 0 || my_rank >= D)
        return -1;
    if (drop_policy != 0 && drop_policy != 1)
        return -1;
    if (drop_policy == 1 && !topk_w && (int64_t)T * k > 0)
        return -1;
    int64_t C = oracle_capacity(T, k, E, cf, min_capacity);
    int32_t *running = calloc((size_t)E, sizeof *running);
    int32_t *position = malloc((size_t)T * k * sizeof *position);
    if (!running || !position) {
        free(running);
        free(position);
        return -2;
    }
    int64_t invalid = 0;
    for (int e = 0; e < E; ++e)
        expert_count[e] = 0;
    /* histogram and token-order positions */
    for (int t = 0; t < T; ++t) {
        for (int s = 0; s < k; ++s) {
            int32_t e = topk_idx[(size_t)t * k + s];
            int repeated = 0;
            for (int s2 = 0; s2 < s; ++s2)
                if (topk_idx[(size_t)t * k + s2] == e)
                    repeated = 1;
            if (e < 0 || e >= E || repeated) {
                position[(size_t)t * k + s] = -1;
                ++invalid;
                continue;
            }
            position[(size_t)t * k + s] = running[e]++;
            expert_count[e]++;
        }
    }
    /* kept counts and offsets */
    int64_t kept_total = 0, max_count = 0;
    int64_t acc = 0;
    for (int e = 0; e < E; ++e) {
        int64_t n = expert_count[e];
        int64_t kept = (C < 0 || n < C) ? n : C;
        expert_kept[e] = (int32_t)kept;
        kept_total += kept;
        if (n > max_count)
            max_count = n;
        expert_offset[e] = (C < 0) ? acc : (int64_t)e * C;
        acc += n;
    }
    int64_t send_rows = (C < 0) ? (int64_t)T * k : (int64_t)E * C;
    expert_offset[E] = (C < 0) ? acc : (int64_t)E * C;
    /* drop policy 1: re-rank the assignments of every overflowing expert */
    if (drop_policy == 1 && C >= 0) {
        int32_t *list = malloc(((size_t)T * k + 1) * sizeof *list);
        int64_t *start = malloc(((size_t)E + 1) * sizeof *start);
        if (!list || !start) {
            free(list);
            free(start);
            free(running);
            free(position);
            return -2;
        }
        start[0] = 0;
        for (int e = 0; e < E; ++e)
            start[e + 1] = start[e] + expert_count[e];
        /* each expert's assignments, in ascending token order */
        for (int64_t a = 0; a < (int64_t)T * k; ++a)
            if (position[a] >= 0)
                list[start[topk_idx[a]] + position[a]] = (int32_t)a;
        g_cmp_w = topk_w;
        g_cmp_k = k;
        for (int e = 0; e < E; ++e) {
            int64_t n = expert_count[e];
            if (n <= C)
                continue; /* everything fits: token-order positions stand */
            int32_t *mine = list + start[e];
            int32_t *ranked = malloc((size_t)n * sizeof *ranked);
            if (!ranked) {
                free(list);
                free(start);
                free(running);
                free(position);
                return -2;
            }
            memcpy(ranked, mine, (size_t)n * sizeof *ranked);
            qsort(ranked, (size_t)n, sizeof *ranked, by_gate_then_token);
            /* mark the C best; then number the kept ones in token order */
            for (int64_t i = 0; i < n; ++i)
                position[ranked[i]] = i < C ? 1 : 0;
            int32_t next = 0;
            for (int64_t i = 0; i < n; ++i) /* dropped: -1, no slot */
                position[mine[i]] = position[mine[i]] == 1 ? next++ : -1;
            free(ranked);
        }
        free(list);
        free(start);
    }
    /* slots and the send buffer: bf16 rows, or [F8] E4M3 rows + scales
     * (pad rows: zero codes, scale 0) */
    const size_t elem = fp8 ? 1 : 2;
    uint8_t *qrow = NULL;
    float qscale = 0.0f;
    if (fp8 && send_buf && !(qrow = malloc((size_t)d))) {
        free(running);
        free(position);
        return -2;
    }
    if (send_buf)
        memset(send_buf, 0, (size_t)send_rows * d * elem);
    if (fp8 && send_buf)
        for (int64_t r = 0; r < send_rows; ++r)
            send_scale[r] = 0.0f;
    for (int t = 0; t < T; ++t) {
        if (qrow)
            oracle_fp8_quantize_rows(1, d, x + (size_t)t * d, qrow, &qscale);
        for (int s = 0; s < k; ++s) {
            int32_t e = topk_idx[(size_t)t * k + s];
            int32_t p = position[(size_t)t * k + s];
            int32_t sl = -1;
            if (p >= 0 && (C < 0 || p < C))
                sl = (int32_t)(expert_offset[e] + p);
            slot[(size_t)t * k + s] = sl;
            if (sl < 0 || !send_buf)
                continue;
            if (fp8) {
                memcpy((uint8_t *)send_buf + (size_t)sl * d, qrow, (size_t)d);
                send_scale[sl] = qscale;
            } else {
                memcpy((uint16_t *)send_buf + (size_t)sl * d, x + (size_t)t * d, (size_t)d * 2);
            }
        }
    }
    free(qrow);
    /* per-rank rows (kept token vectors per destination) */
    int epr = E / D;
    int64_t remote_rows = 0;
    for (int r = 0; r < D; ++r) {
        int64_t rows = 0;
        for (int e = r * epr; e < (r + 1) * epr; ++e)
            rows += expert_kept[e];
        rank_rows[r] = rows;
        if (r != my_rank)
            remote_rows += rows;
    }
    stats[ST_ASSIGNMENTS] = (int64_t)T * k;
    stats[ST_KEPT] = kept_total;
    stats[ST_DROPPED] = (int64_t)T * k - kept_total;
    stats[ST_PADDED] = (C < 0) ? 0 : (int64_t)E * C - kept_total;
    stats[ST_CAPACITY] = C;
    stats[ST_SEND_ROWS] = send_rows;
    /* a dispatched row: d bf16, or [F8] d E4M3 codes plus its fp32 scale */
    const int64_t row_bytes = fp8 ? (int64_t)d + 4 : (int64_t)d * 2;
    stats[ST_DISPATCH_BYTES] = kept_total * row_bytes;
    stats[ST_WIRE_BYTES] = (C < 0) ? kept_total * row_bytes : send_rows * row_bytes;
    stats[ST_REMOTE_BYTES] = remote_rows * row_bytes;
    stats[ST_COMBINE_BYTES] = kept_total * d * 2;
    stats[ST_MAX_COUNT] = max_count;
    stats[ST_INVALID] = invalid;
    free(running);
    free(position);
    return 0;
}

/* ------------------------------------------------------------------ */
/* Step 5: one expert's SwiGLU FFN on n rows.                 [M]      */
/* rows [n, d] bf16; w1, w3 [H, d] bf16; w2 [d, H] bf16; out [n, d].   */
/* g = W1 x, u = W3 x (double), h = bf16(SiLU(g) * u) with             */
/* SiLU(z) = z / (1 + exp(-z)), out = bf16(W2 h).                      */
/*                                                                     */
/* bound (optional, [n, d] double; test infrastructure): how far the   */
/* unrounded result of an fp32 evaluation of the same expert may lie   */
/* from the exact W2 h, given bf16 inputs equal to these, under the    */
/* standard probabilistic model of rounding errors (independent, mean  */
/* zero; Higham and Mary, SIAM J. Sci. Comput. 41(5), 2019): a sum of  */
/* m products in fp32, in any order, is within                         */
/*   G(m) * sum|terms|,  G(m) = exp(L sqrt(m) u + m u^2/(1-u)) - 1,     */
/* of the exact sum, u = 2^-24, L = 8 (failing with probability below  */
/* 2 m exp(-L^2/2) < 3e-10 per sum at m = 14336).  So g and u are      */
/* within Gg = G(d+2) sum|x w1| and Gu (the +2 covers the row scale of */
/* E4M3 rows and a final rounding); SiLU(g) * u, evaluated in fp32     */
/* (exp, add, divide, multiply: 8 u relative allowed), within          */
/*   e = 1.01 (|SiLU'(g) u| Gg + |SiLU(g)| Gu) + Gg Gu + 8 u |v|        */
/* of v = SiLU(g) u, so the fp32 side's h_j is a bf16 value in         */
/* [bf16(v - e), bf16(v + e)], at most s_j = that interval's width     */
/* from this h_j (s_j = 0 unless v_j lies within e_j of a bf16         */
/* rounding boundary).  Which way such an h_j goes is taken as         */
/* independent of the others, so their effect on an output sums to at */
/* most L sqrt(sum (s_j w2_j)^2) (Hoeffding; failing with probability  */
/* below 2 exp(-L^2/2) = 3e-14), and                                   */
/*   bound = L sqrt(sum (s w2)^2) + G(H) (sum|h w2| + sum s|w2|).       */
/* ------------------------------------------------------------------ */
#define BOUND_L 8.0
static double gamma_n(double m)
{
    const double u = ldexp(1.0, -24);
    return exp(BOUND_L * sqrt(m) * u + m * u * u / (1.0 - u)) - 1.0;
}

/* Gate/up half of the expert on one row: h_j = bf16(SiLU(g_j) u_j) for
 * j < H, g = W1 x, u = W3 x in double; with e non-NULL also e_j, the bound
 * on |fp32 evaluation of SiLU(g_j) u_j - SiLU(g_j) u_j| derived above; with
 * spread non-NULL the width s_j of [bf16(v - e), bf16(v + e)]. */
static void gate_up_row(int d, int H, const double *xr, const uint16_t *w1, const uint16_t *w3,
                        double *h, double *e, double *spread)
{
    const double u32 = ldexp(1.0, -24);
    for (int j = 0; j < H; ++j) {
        double g = 0.0, u = 0.0, ag = 0.0, au = 0.0;
        for (int i = 0; i < d; ++i) {
            const double a = xr[i] * bf16_value(w1[(size_t)j * d + i]);
            const double b = xr[i] * bf16_value(w3[(size_t)j * d + i]);
            g += a;
            u += b;
            ag += fabs(a);
            au += fabs(b);
        }
        const double sg = 1.0 / (1.0 + exp(-g));
        const double silu = g * sg;
        const double v = silu * u;
        h[j] = bf16_value(oracle_bf16_from_double(v));
        if (e || spread) {
            const double Gg = gamma_n(d + 2) * ag, Gu = gamma_n(d + 2) * au;
            const double dsilu = sg * (1.0 + g * (1.0 - sg));
            const double ej = 1.01 * (fabs(dsilu * u) * Gg + fabs(silu) * Gu) + Gg * Gu +
                              8.0 * u32 * fabs(v);
            if (e)
                e[j] = ej;
            if (spread)
                spread[j] = bf16_value(oracle_bf16_from_double(v + ej)) -
                            bf16_value(oracle_bf16_from_double(v - ej));
        }
    }
}

/* Down half on one row: out_m = bf16(sum_j h_j W2_mj); with bound non-NULL
 * also the bound on |fp32 evaluation of the sum - exact sum|: for h values
 * shared by both sides (spread == NULL) G(H) sum|h w2|; for h values that
 * may each lie spread_j away on the fp32 side, as derived above. */
static void down_row(int d, int H, const double *h, const double *spread, const uint16_t *w2,
                     uint16_t *out, double *bound)
{
    for (int m = 0; m < d; ++m) {
        double o = 0.0, ao = 0.0, so = 0.0, s2 = 0.0;
        for (int j = 0; j < H; ++j) {
            const double w = bf16_value(w2[(size_t)m * H + j]);
            o += h[j] * w;
            if (bound) {
                ao += fabs(h[j] * w);
                if (spread) {
                    so += spread[j] * fabs(w);
                    s2 += spread[j] * w * spread[j] * w;
                }
            }
        }
        out[m] = oracle_bf16_from_double(o);
        if (bound)
            bound[m] = BOUND_L * sqrt(s2) + gamma_n(H) * (ao + so);
    }
}

/* The row's values: bf16 (codes == NULL) or [F8] E4M3 codes times the row's
 * scale (exact in double). */
static void row_values(int d, int r, const uint16_t *rows, const uint8_t *codes,
                       const float *scales, double *xr)
{
    for (int i = 0; i < d; ++i)
        xr[i] = codes ? oracle_fp8_value(codes[(size_t)r * d + i]) * (double)scales[r]
                      : bf16_value(rows[(size_t)r * d + i]);
}

/* The whole expert on n rows; bound: the end-to-end bound derived above. */
static void expert_ffn_rows(int n, int d, int H, const uint16_t *rows, const uint8_t *codes,
                            const float *scales, const uint16_t *w1, const uint16_t *w3,
                            const uint16_t *w2, uint16_t *out, double *bound)
{
#pragma omp parallel
    {
        double *xr = malloc((size_t)d * sizeof *xr);
        double *h = malloc((size_t)H * sizeof *h);
        double *sp = bound ? malloc((size_t)H * sizeof *sp) : NULL;
#pragma omp for schedule(dynamic, 1)
        for (int r = 0; r < n; ++r) {
            row_values(d, r, rows, codes, scales, xr);
            gate_up_row(d, H, xr, w1, w3, h, NULL, sp);
            down_row(d, H, h, sp, w2, out + (size_t)r * d, bound ? bound + (size_t)r * d : NULL);
        }
        free(xr);
        free(h);
        free(sp);
    }
}

void oracle_expert_ffn(int n, int d, int H, const uint16_t *rows, const uint16_t *w1,
                       const uint16_t *w3, const uint16_t *w2, uint16_t *out, double *bound)
{
    expert_ffn_rows(n, d, H, rows, NULL, NULL, w1, w3, w2, out, bound);
}

/* The same FFN on FP8 rows (codes [n, d], scales [n]).          [F8]  */
void oracle_expert_ffn_fp8(int n, int d, int H, const uint8_t *codes, const float *scales,
                           const uint16_t *w1, const uint16_t *w3, const uint16_t *w2,
                           uint16_t *out, double *bound)
{
    expert_ffn_rows(n, d, H, NULL, codes, scales, w1, w3, w2, out, bound);
}

/* The two halves apart (stage checks on identical inputs).  Gate/up: rows
 * [n, d] bf16 (codes == NULL) or E4M3 codes + scales -> h [n, H] bf16, and
 * bound_h [n, H] (optional): e_j above.  Down: h [n, H] bf16 -> out [n, d],
 * and bound [n, d] (optional): G(H) sum|h w2|.  down(gate_up(x)) is the
 * expert above, bit for bit. */
static void expert_gate_up_rows(int n, int d, int H, const uint16_t *rows, const uint8_t *codes,
                                const float *scales, const uint16_t *w1, const uint16_t *w3,
                                uint16_t *h_out, double *bound_h)
{
#pragma omp parallel
    {
        double *xr = malloc((size_t)d * sizeof *xr);
        double *h = malloc((size_t)H * sizeof *h);
#pragma omp for schedule(dynamic, 1)
        for (int r = 0; r < n; ++r) {
            row_values(d, r, rows, codes, scales, xr);
            gate_up_row(d, H, xr, w1, w3, h, bound_h ? bound_h + (size_t)r * H : NULL, NULL);
            for (int j = 0; j < H; ++j)
                h_out[(size_t)r * H + j] = oracle_bf16_from_double(h[j]);
        }
        free(xr);
        free(h);
    }
}

void oracle_expert_gate_up(int n, int d, int H, const uint16_t *rows, const uint16_t *w1,
                           const uint16_t *w3, uint16_t *h, double *bound_h)
{
    expert_gate_up_rows(n, d, H, rows, NULL, NULL, w1, w3, h, bound_h);
}

void oracle_expert_gate_up_fp8(int n, int d, int H, const uint8_t *codes, const float *scales,
                               const uint16_t *w1, const uint16_t *w3, uint16_t *h,
                               double *bound_h)
{
    expert_gate_up_rows(n, d, H, NULL, codes, scales, w1, w3, h, bound_h);
}

void oracle_expert_down(int n, int d, int H, const uint16_t *h, const uint16_t *w2,
                        uint16_t *out, double *bound)
{
#pragma omp parallel
    {
        double *hr = malloc((size_t)H * sizeof *hr);
#pragma omp for schedule(dynamic, 1)
        for (int r = 0; r < n; ++r) {
            for (int j = 0; j < H; ++j)
                hr[j] = bf16_value(h[(size_t)r * H + j]);
            down_row(d, H, hr, NULL, w2, out + (size_t)r * d, bound ? bound + (size_t)r * d : NULL);
        }
        free(hr);
    }
}

/* ------------------------------------------------------------------ */
/* Step 6: combine.                                 [G][CA][TD][SE]    */
/* y[t] = bf16( sum over kept s, in rank order, of G[t,s] * O[slot]    */
/*              + S[t] ), S the shared expert's output (or nothing).   */
/* A dropped assignment (slot < 0) adds nothing; the residual is the   */
/* caller's.  expert_out [*, d] bf16, slot/topk_w [T, k], shared_out   */
/* [T, d] bf16 or NULL, y [T, d].                                      */
/* ------------------------------------------------------------------ */
void oracle_combine(int T, int d, int k, const uint16_t *expert_out, const int32_t *slot,
                    const float *topk_w, const uint16_t *shared_out, uint16_t *y)
{
#pragma omp parallel for schedule(static)
    for (int t = 0; t < T; ++t) {
        for (int m = 0; m < d; ++m) {
            double acc = 0.0;
            for (int s = 0; s < k; ++s) {
                int32_t sl = slot[(size_t)t * k + s];
                if (sl < 0)
                    continue;
                acc += (double)topk_w[(size_t)t * k + s] *
                       bf16_value(expert_out[(size_t)sl * d + m]);
            }
            if (shared_out)
                acc += bf16_value(shared_out[(size_t)t * d + m]);
            y[(size_t)t * d + m] = oracle_bf16_from_double(acc);
        }
    }
}

int oracle_num_threads(void)
{
#ifdef _OPENMP
    return omp_get_max_threads();
#else
    return 1;
#endif
}
