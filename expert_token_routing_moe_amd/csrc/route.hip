// Router: logits H = x W_g (+ b) on bf16 matrix cores, then KeepTopK and a
// softmax over the kept logits ("Mixture-of-Experts (MoE) Architecture and
// Expert Parallelism", section 2 "The Gating Network Formulation"; the noise
// term is zero at inference).
//
// Logits.  A workgroup owns a BT-token x BE-expert tile of the logits over
// one of S slices of K.  x rows and W_g rows stream through one LDS ring by
// direct-to-LDS loads; W_g is read in the page's own [d, E] layout (each K
// step's rows are one contiguous block of memory), and the matrix-core B
// fragments, which need 8 consecutive K values of one expert, come out of
// the ring by the gfx950 transposing LDS read (ds_read_b64_tr_b16).  bf16
// products are exact in fp32 and accumulate in fp32
// (v_mfma_f32_16x16x32_bf16).
//
// Selection, one wavefront per token, each lane holding a run of
// consecutive experts: k rounds of a wave-wide maximum of order-preserving
// 32-bit value images, the winner being the lowest expert index that holds
// the maximum (one ballot and one lane read), then a softmax over the kept
// logits, optionally within the token's best expert groups.
//
// Every workgroup stores its fp32 partial tile; a second launch, one
// wavefront per token, sums a token's partials in slice order (a fixed
// order: deterministic), adds the bias and selects.  The kernel boundary is
// the device-wide barrier: on this eight-XCD part a release inside the
// kernel means an L2 write-back per workgroup, which measured slower than
// the second launch.  (Selecting inside the logit kernel when one workgroup
// holds whole logit rows measured slower too: its 8 waves select 64 tokens
// one after another, where the second launch gives every token a wave.)
#include <type_traits>

#include "moe_internal.hpp"
#include "ring.hpp"

namespace moe {

int router_epad(int E) { return (E + 63) / 64 * 64; }

// W_g row length as the router reads it: E when E % 8 == 0 (the caller's
// tensor), else E rounded up to 8 (a zero-padded copy in the workspace).
int router_ldw(int E) { return (E + 7) / 8 * 8; }

// Launch shape of the logit GEMM: 64-token tiles of BE experts (taller ones
// when there are many, below), and K cut into S slices when the tiles alone
// leave the chip short of workgroups
// (one per CU for BE = 256, eight waves; two per CU for BE = 128 or 64, four
// waves): as many slices as the chip holds in one round of workgroups, at
// least four K steps each, at most 32 (a launch just past one round would
// run a second round for a few workgroups: at 3072 tokens of DeepSeek-V3
// shape 6 slices made 288 workgroups, 5 make 240).  BE is the widest of
// 256, 128, 64 (dividing E rounded up to 64) whose launch fills the chip,
// or at least half of it in one round when the slice count is not at its
// cap; when none does (few tokens: DeepSeek-V3 decode has one token tile
// and 28 slices), the one with the most workgroups, so that more CUs
// stream W_g.  The K slices do not depend on BE, so neither do the
// logits' bits.  (128-token tiles with twice the slices measured the same
// time at the DeepSeek-V3 prefill shape for twice the partial-sum bytes.)
// T = 0: nothing to split.
struct RouterPlan {
    int be, sk, bt;
};
static RouterPlan router_plan(int T, int E, int d)
{
    const int epad = router_epad(E);
    const int steps = d / 64;
    RouterPlan best{64, 1, 64};
    long long best_wg = -1;
    for (int be = 256; be >= 64; be /= 2) {
        if (epad % be != 0)
            continue;
        const int target = be == 256 ? 256 : 512;
        const long long tiles = (long long)((T + 63) / 64) * (epad / be);
        int sk = 1;
        bool capped = false; // fewer slices than one round would hold
        if (T > 0 && tiles < target) {
            const int fit = (int)(target / tiles);
            const int cap = std::max(1, std::min(steps / 4, 32));
            sk = std::max(1, std::min(fit, cap));
            capped = fit > cap;
        }
        const long long wg = tiles * sk;
        // More tiles than one round of workgroups: taller token tiles (128,
        // and 256 for 256-expert tiles, whose ring holds two of their 64 KB
        // stages), so each reads W_g for more tokens (at T = 32768 every
        // 64-token tile would read all of W_g, 3.7 MB at DeepSeek-V3 shape)
        // and fewer rounds run
        if (T > 0 && be == 256 && tiles > 2LL * target)
            return RouterPlan{be, 1, 256};
        if (T > 0 && tiles > target)
            return RouterPlan{be, 1, 128};
        if (T == 0 || wg >= target || (!capped && 2 * wg >= target))
            return RouterPlan{be, sk, 64};
        if (wg > best_wg) {
            best_wg = wg;
            best = RouterPlan{be, sk, 64};
        }
    }
    return best;
}

int router_ksplit(int T, int E, int d) { return router_plan(T, E, d).sk; }

// The logit kernel always stores partial sums (any T > 0).
bool router_partials(int T, int, int) { return T > 0; }

namespace {

typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));

// Ring slot of W_g piece p (16 bytes, 8 experts) of K row r inside the tile
// row of BPR pieces: p ^ swzb(r).  The four rows one transposing read
// touches per 16-lane group land in four distinct 32-byte slots of one
// 128-byte block, and the groups of a wave in different blocks.
template <int BPR>
__device__ __forceinline__ int swzb(int r)
{
    int s = (r & 3) << 1;
    if constexpr (BPR >= 16)
        s |= ((r >> 3) & 1) << 3;
    if constexpr (BPR >= 32)
        s |= ((r >> 4) & 1) << 4;
    return s;
}

// Order-preserving 32-bit image of a finite fp32 logit: larger image =
// larger logit, -0 and +0 equal, and every image of a real value above 0.
__device__ __forceinline__ uint32_t value_key(float v)
{
    uint32_t u = __float_as_uint(v == 0.f ? 0.f : v); // -0 and +0 compare equal
    return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}
__device__ __forceinline__ float key_value(uint32_t u)
{
    u = (u & 0x80000000u) ? (u & 0x7fffffffu) : ~u;
    return __uint_as_float(u);
}

// v = max(v, v of the lane that DPP control CTRL selects), for the rows in
// ROW_MASK; a lane outside them, or without a source, takes 0 from the move,
// which leaves its own value (0 is the identity of the unsigned maximum, so
// the move folds into one DPP maximum instruction).
template <int CTRL, int ROW_MASK>
__device__ __forceinline__ uint32_t max_dpp(uint32_t v)
{
    const uint32_t o = (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, CTRL, ROW_MASK, 0xF, true);
    return o > v ? o : v;
}

// Maximum over the wavefront, returned in every lane: within each 16-lane row
// by quad permutes and the half-row / row mirrors, across rows by the row
// broadcasts of lanes 15 and 31 (lane 63 then holds the total).
__device__ __forceinline__ uint32_t wave_max_u32(uint32_t v)
{
    v = max_dpp<0xB1, 0xF>(v);  // quad_perm [1, 0, 3, 2]
    v = max_dpp<0x4E, 0xF>(v);  // quad_perm [2, 3, 0, 1]
    v = max_dpp<0x141, 0xF>(v); // row_half_mirror
    v = max_dpp<0x140, 0xF>(v); // row_mirror
    v = max_dpp<0x142, 0xA>(v); // row_bcast:15 into rows 1 and 3
    v = max_dpp<0x143, 0xC>(v); // row_bcast:31 into rows 2 and 3
    return (uint32_t)__builtin_amdgcn_readlane((int)v, 63);
}

// Maximum of a 64-bit key over the wavefront: the largest upper half, then
// the largest lower half among the lanes that hold it.
__device__ __forceinline__ uint64_t wave_max_u64(uint64_t v)
{
    const uint32_t hi = wave_max_u32((uint32_t)(v >> 32));
    const uint32_t lo = wave_max_u32((uint32_t)(v >> 32) == hi ? (uint32_t)v : 0u);
    return ((uint64_t)hi << 32) | lo;
}

// The wave's own LDS operations have completed (lgkmcnt(0)); the compiler
// keeps memory accesses on their side.
__device__ __forceinline__ void lds_wait()
{
    asm volatile("" ::: "memory");
    __builtin_amdgcn_s_waitcnt(0xc07f);
    asm volatile("" ::: "memory");
}

// KeepTopK + softmax of one token by one wavefront.  Lane l holds the
// logits (bias included) of the V consecutive experts l*V .. l*V+V-1 in
// h[0..V); experts >= E are ignored.  Group limit ("MoE Expert Parallelism
// Sizing: Traffic, Capacity, Fabric": at most M nodes per token, Megatron's
// group-limited routing), when G > 1 and M < G: the E experts form G
// contiguous groups; each group's score is its best logit (LDS atomic max
// of the order-preserving key), the M best groups are picked by M wave
// arg-max rounds (ties to the lower group), and the other groups' experts
// are retired before KeepTopK.  gs/allow: this wave's LDS scratch (G
// entries).
template <int V>
__device__ __forceinline__ void topk_softmax_token(const float (&h)[V], int E, int k, int G,
                                                   int M, uint32_t *gs, uint8_t *allow,
                                                   int32_t *__restrict__ idx_row,
                                                   float *__restrict__ w_row)
{
    const int lane = threadIdx.x & 63;
    // order-preserving 32-bit image of each logit; 0 (below every real
    // value) marks experts past E and retired ones
    uint32_t vk[V];
#pragma unroll
    for (int j = 0; j < V; ++j) {
        const int e = lane * V + j;
        vk[j] = e < E ? value_key(h[j]) : 0u;
    }
    if (G > 1 && M < G) {
        const int per = E / G;
        for (int g = lane; g < G; g += 64) {
            gs[g] = 0u; // below every real score
            allow[g] = 0;
        }
        lds_wait();
#pragma unroll
        for (int j = 0; j < V; ++j) {
            const int e = lane * V + j;
            if (e < E)
                atomicMax(&gs[e / per], vk[j]);
        }
        lds_wait();
        for (int r = 0; r < M; ++r) {
            uint64_t best = 0;
            for (int g = lane; g < G; g += 64) {
                const uint64_t gk = ((uint64_t)gs[g] << 32) | (uint32_t)(G - 1 - g);
                best = (gs[g] != 0u && gk > best) ? gk : best;
            }
            const int gw = G - 1 - (int)(uint32_t)(wave_max_u64(best) & 0xffffffffu);
            if (lane == 0) {
                gs[gw] = 0u; // retired
                allow[gw] = 1;
            }
            lds_wait();
        }
#pragma unroll
        for (int j = 0; j < V; ++j) {
            const int e = lane * V + j;
            if (e < E && !allow[e / per])
                vk[j] = 0;
        }
    }
    // k rounds: the wave-wide maximum of the lanes' best values; the lowest
    // lane holding it holds the lowest expert with that value (lanes own
    // consecutive experts), and within the lane the lowest register holding
    // it (ties to the lower index); the winner is retired.  Rank s's expert
    // and logit stay in lane s % 64, register s / 64, until the end.
    int my_e[V];
    float my_v[V];
#pragma unroll
    for (int j = 0; j < V; ++j) {
        my_e[j] = 0;
        my_v[j] = 0.f;
    }
    float hmax = 0.f;
    // one round: the winner's expert e and logit v; the winner retired
    auto select_one = [&](int &e, float &v) {
        uint32_t head = vk[0];
#pragma unroll
        for (int j = 1; j < V; ++j)
            head = vk[j] > head ? vk[j] : head;
        const uint32_t win = wave_max_u32(head);
        const int wl = (int)__builtin_ctzll(__ballot(head == win));
        int jpos = V - 1;
#pragma unroll
        for (int j = V - 2; j >= 0; --j)
            jpos = vk[j] == win ? j : jpos;
        const int jw = __builtin_amdgcn_readlane(jpos, wl);
        const bool mine = lane == wl;
#pragma unroll
        for (int j = 0; j < V; ++j)
            if (j == jw)
                vk[j] = mine ? 0u : vk[j];
        e = wl * V + jw;
        v = key_value(win);
    };
    if (k <= 64) {
        for (int s = 0; s < k; ++s) {
            int e;
            float v;
            select_one(e, v);
            if (s == 0)
                hmax = v;
            const bool rec = lane == s;
            my_e[0] = rec ? e : my_e[0];
            my_v[0] = rec ? v : my_v[0];
        }
    } else {
        for (int s = 0; s < k; ++s) {
            int e;
            float v;
            select_one(e, v);
            if (s == 0)
                hmax = v;
            const bool rec = lane == (s & 63);
            const int r = s >> 6;
#pragma unroll
            for (int j = 0; j < V; ++j)
                if (j == r) {
                    my_e[j] = rec ? e : my_e[j];
                    my_v[j] = rec ? v : my_v[j];
                }
        }
    }
    // softmax over the kept logits, max-subtracted: every lane takes the
    // exponentials of its ranks, the denominator sums them in rank order
    float p[V];
#pragma unroll
    for (int j = 0; j < V; ++j)
        p[j] = (j * 64 < k && j * 64 + lane < k) ? expf(my_v[j] - hmax) : 0.f;
    float denom = 0.f;
    for (int s = 0; s < k; ++s) {
        const int r = s >> 6;
        float ps = 0.f;
#pragma unroll
        for (int j = 0; j < V; ++j)
            if (j == r)
                ps = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(p[j]), s & 63));
        denom += ps;
    }
#pragma unroll
    for (int j = 0; j < V; ++j) {
        const int s = j * 64 + lane;
        if (j * 64 < k && s < k) {
            idx_row[s] = my_e[j];
            w_row[s] = p[j] / denom;
        }
    }
}

// Selection on caller-given logits: one wavefront per token.
template <int V>
__global__ __launch_bounds__(256) void topk_softmax_kernel(const float *__restrict__ logits,
                                                           int32_t *__restrict__ topk_idx,
                                                           float *__restrict__ topk_w, int T,
                                                           int E, int k, int G, int M)
{
    __shared__ uint32_t s_gscore[4][kMaxExperts];
    __shared__ uint8_t s_allow[4][kMaxExperts];
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const int t = blockIdx.x * 4 + wave;
    if (t >= T)
        return;
    float h[V];
#pragma unroll
    for (int j = 0; j < V; ++j) {
        const int e = lane * V + j;
        h[j] = e < E ? logits[(size_t)t * E + e] : 0.f;
    }
    topk_softmax_token<V>(h, E, k, G, M, s_gscore[wave], s_allow[wave], topk_idx + (size_t)t * k,
                          topk_w + (size_t)t * k);
}

struct RouteArgs {
    const uint16_t *x;        // [T, d] bf16
    const uint16_t *wg;       // [d, ldw] bf16 (ldw % 8 == 0, ldw >= E)
    const float *bias;        // [E] or null
    float *logits_out;        // [T, E] or null
    int32_t *topk_idx;        // [T, k]
    float *topk_w;            // [T, k]
    float *partial;           // [S, T, E_pad] fp32 partial logits
    int T, d, E, ldw, epad, k, G, M;
    int n_tt, n_et, S, total;
};

// The logit GEMM.  BT tokens x BE experts x one K slice per workgroup, stored
// as an fp32 partial tile.
template <int BT, int RBK, int BE, int RRING, int MINB, int WM, int WN>
__global__ __launch_bounds__(WM * WN * 64, MINB) void route_logits_kernel(RouteArgs a)
{
    constexpr int NW = WM * WN;                  // waves per workgroup
    constexpr int RC = RBK / 8, RPI = 64 / RC;   // x: pieces per row, rows per load
    constexpr int A_PW = BT / RPI / NW;          // x loads per wave per stage
    constexpr int BPR = BE / 8;                  // W_g: pieces per tile row
    constexpr int BRPL = 64 / BPR;               // W_g rows per wave-wide load
    constexpr int B_PW = RBK / BRPL / NW;        // W_g loads per wave per stage
    static_assert(A_PW * RPI * NW == BT && B_PW * BRPL * NW == RBK, "whole loads per wave");
    constexpr int A_BYTES = BT * RBK * 2, STAGE = A_BYTES + RBK * BE * 2;
    constexpr int NS = RRING / STAGE < 8 ? RRING / STAGE : 8;
    static_assert(NS >= 2, "two stages fit");
    constexpr int WTT = BT / WM, WTE = BE / WN;  // wave tile
    constexpr int RT = WTT / 16, CT = WTE / 16;
    __shared__ __attribute__((aligned(1024))) char smem[RRING];

    const int w = xcd_remap(blockIdx.x, a.total);
    if (w < 0)
        return;
    // work order: K slice, then token tile, then expert tile.  The XCD remap
    // gives each XCD a contiguous range, so the workgroups of one XCD share
    // one slice of W_g in their L2 while each streams its own x rows.
    const int et = w % a.n_et;
    const int tt = (w / a.n_et) % a.n_tt;
    const int sk = w / (a.n_et * a.n_tt);
    const int t0 = tt * BT, e0 = et * BE;
    const int T = a.T, d = a.d, ldw = a.ldw;
    // slices are cut on 64-deep boundaries, so the sum over K is taken in
    // the same order whatever the step depth
    const int steps = d / 64, spm = 64 / RBK;
    const int s_lo = steps * sk / a.S * spm, s_hi = steps * (sk + 1) / a.S * spm;
    const int nsteps = s_hi - s_lo;

    const int tid = threadIdx.x, lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int wt = wave / WN, we = wave % WN;

    // Load j of wave w fills ring bytes [(NW*j + w) * 1 KB, +1 KB) of its
    // region.  x: lane l writes piece l % 8 of row l / 8 (source piece
    // swizzled).  W_g: lane l writes slot l % BPR of K row l / BPR, i.e.
    // source piece (l % BPR) ^ swzb(row); pieces past the row's end (the
    // last tile when E_pad > ldw) read piece 0 instead (never selected).
    const uint16_t *asrc[A_PW];
    const uint16_t *bsrc[B_PW];
#pragma unroll
    for (int j = 0; j < A_PW; ++j) {
        const int r = (NW * j + wave) * RPI + lane / RC;
        const int piece = (lane % RC) ^ swz<RC>(r);
        const int t = (t0 + r < T) ? t0 + r : t0; // rows past T read row t0 (never stored)
        asrc[j] = a.x + (size_t)t * d + (size_t)s_lo * RBK + piece * 8;
    }
#pragma unroll
    for (int j = 0; j < B_PW; ++j) {
        const int r = (NW * j + wave) * BRPL + lane / BPR;
        const int piece = (lane % BPR) ^ swzb<BPR>(r);
        const int e = e0 + piece * 8 < ldw ? e0 + piece * 8 : 0;
        bsrc[j] = a.wg + ((size_t)s_lo * RBK + r) * ldw + e;
    }
    const uint32_t lds_base = (uint32_t)(uintptr_t)(LDS_AS char *)smem;
    auto issue = [&](int step, int slot) {
        const uint32_t st = lds_base + slot * STAGE;
#pragma unroll
        for (int j = 0; j < A_PW; ++j)
            dma16(asrc[j] + step * RBK, st + (NW * j + wave) * 1024);
#pragma unroll
        for (int j = 0; j < B_PW; ++j)
            dma16(bsrc[j] + (size_t)step * RBK * ldw, st + A_BYTES + (NW * j + wave) * 1024);
    };

    floatx4 acc[RT][CT];
#pragma unroll
    for (int i = 0; i < RT; ++i)
#pragma unroll
        for (int j = 0; j < CT; ++j)
            acc[i][j] = floatx4{0.f, 0.f, 0.f, 0.f};

    for (int u = 0; u < NS - 1 && u < nsteps; ++u)
        issue(u, u);
    LDS_AS char *lds = (LDS_AS char *)smem;
    for (int st = 0; st < nsteps; ++st) {
        const int ahead = min(NS - 2, nsteps - 1 - st);
        wait_vmcnt(ahead * (A_PW + B_PW));
        ring_barrier();
        if (st + NS - 1 < nsteps)
            issue(st + NS - 1, (st + NS - 1) % NS);
        const int As = (st % NS) * STAGE;
        const int Bs = As + A_BYTES;
#pragma unroll
        for (int kc = 0; kc < RC; kc += 4) {
            bf16x8 av[RT], bv[CT];
            const int piece = kc + (lane >> 4);
#pragma unroll
            for (int i = 0; i < RT; ++i) {
                const int r = wt * WTT + i * 16 + (lane & 15);
                av[i] = *reinterpret_cast<const LDS_AS bf16x8 *>(
                    lds + As + r * (RBK * 2) + ((piece ^ swz<RC>(r)) << 4));
            }
            // B fragment of expert column n = n0 + (lane & 15): lane group
            // g = lane / 16 needs K rows 8g .. 8g+7 of this 32-deep half.  A
            // transposing read takes, per 16-lane group, four K rows of 16
            // experts (source lane jj reads row jj / 4, experts 4 (jj % 4)
            // .. +3) and hands lane i the four K values of expert i.
            const int grp = lane >> 4, jj = lane & 15;
#pragma unroll
            for (int j = 0; j < CT; ++j) {
                const int n0 = we * WTE + j * 16;
                const int p = (n0 >> 3) + ((jj & 3) >> 1);
                const int half = (jj & 1) * 8;
                bf16x4 lo, hi;
                {
                    const int r = kc * 8 + grp * 8 + (jj >> 2);
                    lo = __builtin_amdgcn_ds_read_tr16_b64_v4bf16(reinterpret_cast<LDS_AS bf16x4 *>(
                        lds + Bs + r * (BE * 2) + ((p ^ swzb<BPR>(r)) << 4) + half));
                }
                {
                    const int r = kc * 8 + grp * 8 + 4 + (jj >> 2);
                    hi = __builtin_amdgcn_ds_read_tr16_b64_v4bf16(reinterpret_cast<LDS_AS bf16x4 *>(
                        lds + Bs + r * (BE * 2) + ((p ^ swzb<BPR>(r)) << 4) + half));
                }
                bv[j] = __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7);
            }
#pragma unroll
            for (int i = 0; i < RT; ++i)
#pragma unroll
                for (int j = 0; j < CT; ++j)
                    acc[i][j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(av[i], bv[j], acc[i][j],
                                                                         0, 0, 0);
        }
    }

    // D layout of a 16x16 MFMA tile: lane holds rows 4*(lane/16)+q, column
    // lane%16.
    // partial tile -> [sk, t, e0 .. e0 + BE) of the [S, T, E_pad] sums,
    // 64-byte row pieces straight from the accumulators
    float *out = a.partial + (size_t)sk * T * a.epad;
#pragma unroll
    for (int i = 0; i < RT; ++i)
#pragma unroll
        for (int q = 0; q < 4; ++q) {
            const int t = t0 + wt * WTT + i * 16 + 4 * (lane >> 4) + q;
            if (t < T)
#pragma unroll
                for (int j = 0; j < CT; ++j)
                    out[(size_t)t * a.epad + e0 + we * WTE + j * 16 + (lane & 15)] =
                        acc[i][j][q];
        }
}

// Sum of the S partial logits of a token in slice order (loads in batches
// of SB slices, every load of a batch in flight together), plus the bias,
// then selection: one wavefront per token.
template <int V, int SB>
__global__ __launch_bounds__(256) void route_select_kernel(RouteArgs a)
{
    __shared__ uint32_t s_gscore[4][kMaxExperts];
    __shared__ uint8_t s_allow[4][kMaxExperts];
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const int t = blockIdx.x * 4 + wave;
    if (t >= a.T)
        return;
    const int S = a.S, E = a.E, epad = a.epad;
    // lane l sums experts l*V .. l*V+V-1: V consecutive floats of each
    // slice's row (16-byte loads when V >= 4; every row holds E_pad = 64 V)
    float h[V];
    for (int s0 = 0; s0 < S; s0 += SB) {
        float pv[SB][V];
#pragma unroll
        for (int u = 0; u < SB; ++u) {
            const float *src = a.partial + ((size_t)(s0 + u) * a.T + t) * epad + lane * V;
            if constexpr (V % 4 == 0) {
#pragma unroll
                for (int q = 0; q < V / 4; ++q) {
                    const float4 f = s0 + u < S ? reinterpret_cast<const float4 *>(src)[q]
                                                : make_float4(0.f, 0.f, 0.f, 0.f);
                    pv[u][4 * q] = f.x;
                    pv[u][4 * q + 1] = f.y;
                    pv[u][4 * q + 2] = f.z;
                    pv[u][4 * q + 3] = f.w;
                }
            } else {
#pragma unroll
                for (int j = 0; j < V; ++j)
                    pv[u][j] = s0 + u < S ? src[j] : 0.f;
            }
        }
#pragma unroll
        for (int u = 0; u < SB; ++u)
#pragma unroll
            for (int j = 0; j < V; ++j)
                if (s0 + u < S)
                    h[j] = s0 + u == 0 ? pv[u][j] : h[j] + pv[u][j];
    }
#pragma unroll
    for (int j = 0; j < V; ++j) {
        const int e = lane * V + j;
        if (e < E) {
            if (a.bias)
                h[j] += a.bias[e];
            if (a.logits_out)
                a.logits_out[(size_t)t * E + e] = h[j];
        }
    }
    topk_softmax_token<V>(h, E, a.k, a.G, a.M, s_gscore[wave], s_allow[wave],
                          a.topk_idx + (size_t)t * a.k, a.topk_w + (size_t)t * a.k);
}

// W_g [d, E] -> [d, ldw] with zero columns E .. ldw-1 (E % 8 != 0 only).
__global__ __launch_bounds__(256) void pad_wg_kernel(const uint16_t *__restrict__ wg,
                                                     uint16_t *__restrict__ out, int d, int E,
                                                     int ldw)
{
    const long long i = (long long)blockIdx.x * 256 + threadIdx.x;
    if (i >= (long long)d * ldw)
        return;
    const int r = (int)(i / ldw), e = (int)(i % ldw);
    out[i] = e < E ? wg[(size_t)r * E + e] : (uint16_t)0;
}

hipError_t launch_topk(const Dims &dm, const float *logits, int32_t *topk_idx, float *topk_w,
                       hipStream_t st)
{
    if (dm.T == 0)
        return hipSuccess;
    const int blocks = (dm.T + 3) / 4;
    const int V = (dm.E + 63) / 64;
#define MOE_TOPK(VV)                                                                       \
    topk_softmax_kernel<VV><<<blocks, 256, 0, st>>>(logits, topk_idx, topk_w, dm.T, dm.E, \
                                                   dm.k, dm.n_groups, dm.group_limit)
    if (V <= 1)
        MOE_TOPK(1);
    else if (V <= 2)
        MOE_TOPK(2);
    else if (V <= 4)
        MOE_TOPK(4);
    else if (V <= 8)
        MOE_TOPK(8);
    else
        MOE_TOPK(16);
#undef MOE_TOPK
    return hipGetLastError();
}

} // namespace

hipError_t launch_route(const Dims &dm, const uint16_t *x, const uint16_t *w_gate,
                        const float *bias, float *logits_out, int32_t *topk_idx, float *topk_w,
                        char *ws, const Workspace &wl, hipStream_t st)
{
    if (dm.T == 0)
        return hipSuccess;
    const int T = dm.T, E = dm.E, d = dm.d;
    const int ldw = router_ldw(E);
    const uint16_t *wg = w_gate;
    if (ldw != E) {
        uint16_t *pad = reinterpret_cast<uint16_t *>(ws + wl.wg_pad);
        const long long n = (long long)d * ldw;
        pad_wg_kernel<<<(unsigned)((n + 255) / 256), 256, 0, st>>>(w_gate, pad, d, E, ldw);
        const hipError_t e = hipGetLastError();
        if (e != hipSuccess)
            return e;
        wg = pad;
    }
    RouteArgs a{};
    a.x = x;
    a.wg = wg;
    a.bias = bias;
    a.logits_out = logits_out;
    a.topk_idx = topk_idx;
    a.topk_w = topk_w;
    a.partial = reinterpret_cast<float *>(ws + wl.logits);
    a.T = T;
    a.d = d;
    a.E = E;
    a.ldw = ldw;
    a.epad = router_epad(E);
    a.k = dm.k;
    a.G = dm.n_groups;
    a.M = dm.group_limit;
    const RouterPlan plan = router_plan(T, E, d);
    const int be = plan.be;
    a.S = plan.sk;
    a.n_tt = (T + plan.bt - 1) / plan.bt;
    a.n_et = a.epad / be;
    a.total = a.n_tt * a.n_et * a.S;
#define MOE_LOGITS(BT)                                                                       \
    if (be == 256)                                                                           \
        route_logits_kernel<BT, 64, 256, 156 * 1024, 1, 2, 4>                                \
            <<<xcd_grid(a.total), 512, 0, st>>>(a);                                          \
    else if (be == 128)                                                                      \
        route_logits_kernel<BT, 64, 128, 78 * 1024, 2, 2, 2>                                 \
            <<<xcd_grid(a.total), 256, 0, st>>>(a);                                          \
    else                                                                                     \
        route_logits_kernel<BT, 64, 64, 78 * 1024, 2, 2, 2><<<xcd_grid(a.total), 256, 0, st>>>(a);
    if (plan.bt == 256) {
        route_logits_kernel<256, 64, 256, 156 * 1024, 1, 2, 4>
            <<<xcd_grid(a.total), 512, 0, st>>>(a);
    } else if (plan.bt == 128) {
        MOE_LOGITS(128)
    } else {
        MOE_LOGITS(64)
    }
#undef MOE_LOGITS
    hipError_t e = hipGetLastError();
    if (e != hipSuccess)
        return e;
    const int blocks = (T + 3) / 4;
    const int V = a.epad / 64;
    // every slice's loads in flight together when the slices are many (up
    // to 32: DeepSeek-V3 decode has 28) and a lane's experts few; else
    // batches of 8
    const bool one_batch = a.S > 8 && V <= 4;
#define MOE_SEL(VV, SB) route_select_kernel<VV, SB><<<blocks, 256, 0, st>>>(a)
    if (V <= 1)
        one_batch ? MOE_SEL(1, 32) : MOE_SEL(1, 8);
    else if (V <= 2)
        one_batch ? MOE_SEL(2, 32) : MOE_SEL(2, 8);
    else if (V <= 4)
        one_batch ? MOE_SEL(4, 32) : MOE_SEL(4, 8);
    else if (V <= 8)
        MOE_SEL(8, 8);
    else
        MOE_SEL(16, 8);
#undef MOE_SEL
    return hipGetLastError();
}

hipError_t launch_topk_softmax(const Dims &dm, const float *logits, int32_t *topk_idx,
                               float *topk_w, hipStream_t st)
{
    return launch_topk(dm, logits, topk_idx, topk_w, st);
}

} // namespace moe
