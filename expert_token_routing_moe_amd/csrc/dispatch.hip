// Dispatch: per-expert histogram, capacity, token-order positions and the
// send buffer laid out as the dispatch all-to-all sends it.
//
// Sources: "EP Math -- Expert Parallelism (MoE)", sections "Notation"
// (T*k assignments per device), "Capacity factor" (C = f*T*k/E rounded up,
// static [E, C, d] buffer, pads up to C), "Token drop" (overflow beyond C is
// dropped), "Placing experts across devices" (E/D whole experts per rank);
// "MoE Expert Parallelism Sizing: Traffic, Capacity, Fabric", "Capacity
// semantics decide what crosses the wire" (drop before the exchange) and
// "First-order dispatch and combine bytes" (one input chunk per destination).
//
// Three kernels, no host synchronisation, deterministic:
//  1. count: a workgroup per chunk of 256 tokens builds, in LDS, one 256-bit
//     token bitmap per expert (atomicOr, order-free).  The in-chunk position
//     of assignment (t, s) is the popcount of its expert's bitmap below t,
//     which is exactly the number of earlier tokens of the chunk routed to
//     the same expert.  Writes per-chunk counts and the in-chunk positions.
//  2. scan: one workgroup scans the chunk counts of every expert (giving the
//     chunk bases and n_e), applies the capacity, forms the expert offsets,
//     the per-rank rows and the counters.
//  3. permute: a wavefront per token (two or four, each over a share of the
//     row, when there are few tokens) turns positions into slots, reads the
//     token row once and writes it to each kept slot with 16-byte stores;
//     extra workgroups zero the pad rows of capacity mode.
//
// Drop by gate value (drop policy 1, capacity mode; "MoE Expert Parallelism
// Sizing: Traffic, Capacity, Fabric", "Capacity semantics decide what
// crosses the wire": overflow is dropped by selected probability) adds two
// kernels between 2 and 3:
//  a. group: every valid assignment writes its index into its expert's
//     segment of a by-expert list, at its token-order position.
//  b. select: a workgroup per expert.  If the expert holds more than C
//     assignments, a radix select over the gate values finds the C-th
//     largest one exactly; equal gates at that boundary go to the lower
//     tokens, i.e. the first ones in the token-ordered list.  The kept
//     assignments are then numbered in list (token) order by a block scan,
//     and the final in-expert positions replace the in-chunk ones.
// The counts do not change, so the scan's offsets and counters stand.
#include "moe_internal.hpp"

namespace moe {
namespace {

constexpr int kWords = kChunk / 32; // bitmap words per expert

// An entry is valid iff it lies in [0, E) and does not repeat an expert
// already listed earlier for the same token.
__device__ __forceinline__ bool entry_valid(const int32_t *row, int s, int E)
{
    const int32_t e = row[s];
    if (e < 0 || e >= E)
        return false;
    for (int s2 = 0; s2 < s; ++s2)
        if (row[s2] == e)
            return false;
    return true;
}

// KM > 0: k <= KM, and a token's k expert ids are loaded once into registers
// (all loads in flight together), so the validity checks and the bitmap
// updates run on registers; KM == 0: any k, read from memory as needed.
template <int KM>
__global__ __launch_bounds__(kChunk) void count_kernel(const int32_t *__restrict__ topk_idx,
                                                       int T, int k, int E,
                                                       int32_t *__restrict__ pos_in_chunk,
                                                       int32_t *__restrict__ chunk_counts,
                                                       int32_t *__restrict__ chunk_invalid)
{
    extern __shared__ uint32_t bm[]; // [E][kWords]
    __shared__ int s_invalid;
    const int i = threadIdx.x;
    const int chunk = blockIdx.x;
    const int t = chunk * kChunk + i;
    const int32_t *row = topk_idx + (size_t)t * k;
    int32_t ids[KM > 0 ? KM : 1];
    bool ok[KM > 0 ? KM : 1];
    if constexpr (KM > 0) {
#pragma unroll
        for (int s = 0; s < KM; ++s)
            ids[s] = (t < T && s < k) ? row[s] : -1;
#pragma unroll
        for (int s = 0; s < KM; ++s) {
            ok[s] = s < k && ids[s] >= 0 && ids[s] < E;
#pragma unroll
            for (int s2 = 0; s2 < s; ++s2)
                ok[s] = ok[s] && ids[s2] != ids[s];
        }
    }
    for (int w = i; w < E * kWords; w += kChunk)
        bm[w] = 0u;
    if (i == 0)
        s_invalid = 0;
    __syncthreads();
    const uint32_t bit = 1u << (i & 31);
    if (t < T) {
        if constexpr (KM > 0) {
#pragma unroll
            for (int s = 0; s < KM; ++s)
                if (ok[s])
                    atomicOr(&bm[ids[s] * kWords + (i >> 5)], bit);
        } else {
            for (int s = 0; s < k; ++s)
                if (entry_valid(row, s, E))
                    atomicOr(&bm[row[s] * kWords + (i >> 5)], bit);
        }
    }
    __syncthreads();
    if (t < T) {
        int invalid = 0;
        auto position = [&](int e) { // earlier tokens of the chunk routed to e
            const uint32_t *m = bm + e * kWords;
            int p = __popc(m[i >> 5] & (bit - 1u));
            for (int w = 0; w < (i >> 5); ++w)
                p += __popc(m[w]);
            return p;
        };
        if constexpr (KM > 0) {
#pragma unroll
            for (int s = 0; s < KM; ++s) {
                if (s >= k)
                    break;
                const int32_t p = ok[s] ? position(ids[s]) : -1;
                invalid += ok[s] ? 0 : 1;
                pos_in_chunk[(size_t)t * k + s] = p;
            }
        } else {
            for (int s = 0; s < k; ++s) {
                int32_t p = -1;
                if (entry_valid(row, s, E))
                    p = position(row[s]);
                else
                    ++invalid;
                pos_in_chunk[(size_t)t * k + s] = p;
            }
        }
        if (invalid)
            atomicAdd(&s_invalid, invalid);
    }
    for (int e = i; e < E; e += kChunk) {
        int c = 0;
#pragma unroll
        for (int w = 0; w < kWords; ++w)
            c += __popc(bm[e * kWords + w]);
        chunk_counts[(size_t)chunk * E + e] = c;
    }
    __syncthreads();
    if (i == 0)
        chunk_invalid[chunk] = s_invalid;
}

// Outputs of the scan over chunks and experts.
struct ScanOut {
    int32_t *chunk_base, *expert_count, *expert_kept, *expert_offset, *rank_rows;
    moe_stats *stats;
    int32_t *all_offset; // drop policy 1 only (else null)
};

// The scan, by one workgroup of 1024 threads (thread e owns expert e):
// chunk bases (exclusive scan of the chunk counts of each expert, in chunk
// order), n_e and the kept counts, the expert offsets (an exclusive scan
// over experts when dropless, e*C otherwise), the per-rank rows and the
// counters.  counts: [nchunks, E], global or LDS memory; inv: this thread's
// share of the invalid entries.
__device__ __forceinline__ void scan_block(int T, int k, int E, int D, int my_rank, int d,
                                           int fp8, long long C, int nchunks,
                                           const int32_t *counts, int inv, const ScanOut &o)
{
    __shared__ int32_t s_rank[kMaxExperts];
    __shared__ int32_t s_wave_sum[kMaxExperts / 64];
    __shared__ int s_kept_total, s_max, s_remote, s_invalid;
    const int e = threadIdx.x;
    const int lane = e & 63, wave = e >> 6;
    if (e == 0) {
        s_kept_total = 0;
        s_max = 0;
        s_remote = 0;
        s_invalid = 0;
    }
    int n = 0, kept = 0;
    if (e < E) {
        // the chunk counts are loaded 16 at a time, all in flight together
        for (int c0 = 0; c0 < nchunks; c0 += 16) {
            int cv[16];
#pragma unroll
            for (int u = 0; u < 16; ++u)
                cv[u] = c0 + u < nchunks ? counts[(size_t)(c0 + u) * E + e] : 0;
#pragma unroll
            for (int u = 0; u < 16; ++u)
                if (c0 + u < nchunks) {
                    o.chunk_base[(size_t)(c0 + u) * E + e] = n;
                    n += cv[u];
                }
        }
        kept = (C < 0 || n < C) ? n : (int)C;
        o.expert_count[e] = n;
        o.expert_kept[e] = kept;
    }
    // exclusive scan of n over experts (dropless offsets): wave scan + wave totals
    int incl = n;
#pragma unroll
    for (int off = 1; off < 64; off <<= 1) {
        const int v = __shfl_up(incl, off, 64);
        if (lane >= off)
            incl += v;
    }
    if (lane == 63)
        s_wave_sum[wave] = incl;
    __syncthreads();
    int wave_base = 0;
#pragma unroll
    for (int w = 0; w < kMaxExperts / 64; ++w) // all reads in flight together
        wave_base += w < wave ? s_wave_sum[w] : 0;
    const int excl = wave_base + incl - n;
    if (e < E)
        o.expert_offset[e] = (C < 0) ? excl : (int)((long long)e * C);
    if (o.all_offset && e < E)
        o.all_offset[e] = excl; // where expert e's assignments start in the by-expert list
    if (e == E - 1)
        o.expert_offset[E] = (C < 0) ? excl + n : (int)((long long)E * C);
    // reductions: within each wave first (one LDS atomic per wave)
    int kt = kept, mx = n;
#pragma unroll
    for (int off = 32; off >= 1; off >>= 1) {
        kt += __shfl_xor(kt, off, 64);
        mx = max(mx, __shfl_xor(mx, off, 64));
        inv += __shfl_xor(inv, off, 64);
    }
    if (lane == 0) {
        atomicAdd(&s_kept_total, kt);
        atomicMax(&s_max, mx);
        atomicAdd(&s_invalid, inv);
    }
    const int epr = E / D;
    if (e < D)
        s_rank[e] = 0;
    __syncthreads();
    if (e < E && kept)
        atomicAdd(&s_rank[e / epr], kept);
    __syncthreads();
    for (int r = e; r < D; r += kMaxExperts) {
        const int rows = s_rank[r];
        o.rank_rows[r] = rows;
        if (r != my_rank)
            atomicAdd(&s_remote, rows);
    }
    __syncthreads();
    if (e == 0) {
        const long long kt = s_kept_total;
        const long long assignments = (long long)T * k;
        const long long send_rows = (C < 0) ? assignments : (long long)E * C;
        moe_stats st;
        st.assignments = assignments;
        st.kept = kt;
        st.dropped = assignments - kt;
        st.padded = (C < 0) ? 0 : (long long)E * C - kt;
        st.capacity = C;
        st.send_rows = send_rows;
        // a dispatched row: d bf16, or d E4M3 codes plus its fp32 scale
        const long long row_bytes = fp8 ? (long long)d + 4 : (long long)d * 2;
        st.dispatch_bytes = kt * row_bytes;
        st.dispatch_wire_bytes = (C < 0) ? kt * row_bytes : send_rows * row_bytes;
        st.dispatch_remote_bytes = (long long)s_remote * row_bytes;
        st.combine_bytes = kt * d * 2;
        st.max_expert_count = s_max;
        st.invalid_index = s_invalid;
        *o.stats = st;
    }
}

// Single workgroup of 1024 threads: the scan of the count kernel's chunk
// counts.
__global__ __launch_bounds__(kMaxExperts) void scan_kernel(
    int T, int k, int E, int D, int my_rank, int d, int fp8, long long C, int nchunks,
    const int32_t *__restrict__ chunk_counts, const int32_t *__restrict__ chunk_invalid,
    ScanOut o)
{
    int inv = 0;
    for (int c = threadIdx.x; c < nchunks; c += kMaxExperts)
        inv += chunk_invalid[c];
    scan_block(T, k, E, D, my_rank, d, fp8, C, nchunks, chunk_counts, inv, o);
}

// Count and scan in one workgroup of 1024 threads, for small shapes whose
// chunk bitmaps all fit in LDS (nchunks * E <= kFusedCells) and whose routing
// entries fit in registers (T <= 1024, k <= KM: thread t takes token t and
// loads all its entries before using any): the count kernel's per-chunk
// token bitmaps for every chunk at once, their popcounts as the chunk
// counts, the scan, then the in-chunk positions.  Same outputs as
// count_kernel + scan_kernel, in one launch.
constexpr int kFusedCells = 4096;
template <int KM>
__global__ __launch_bounds__(1024) void count_scan_kernel(
    const int32_t *__restrict__ topk_idx, int T, int k, int E, int D, int my_rank, int d,
    int fp8, long long C, int nchunks, int32_t *__restrict__ pos_in_chunk, ScanOut o)
{
    __shared__ uint32_t s_bm[kFusedCells * kWords]; // [nchunks][E][kWords]
    __shared__ int32_t s_cnt[kFusedCells];          // [nchunks][E]
    const int t = threadIdx.x;
    const int cells = nchunks * E;
    int32_t ids[KM];
    bool ok[KM];
#pragma unroll
    for (int s = 0; s < KM; ++s)
        ids[s] = (t < T && s < k) ? topk_idx[(size_t)t * k + s] : -1;
    for (int w = t; w < cells * kWords; w += 1024)
        s_bm[w] = 0u;
    int invalid = 0;
#pragma unroll
    for (int s = 0; s < KM; ++s) {
        ok[s] = ids[s] >= 0 && ids[s] < E;
#pragma unroll
        for (int s2 = 0; s2 < s; ++s2)
            ok[s] = ok[s] && ids[s2] != ids[s];
        invalid += (t < T && s < k && !ok[s]) ? 1 : 0;
    }
    __syncthreads();
    {
        uint32_t *bm = s_bm + (size_t)(t / kChunk) * E * kWords + ((t % kChunk) >> 5);
#pragma unroll
        for (int s = 0; s < KM; ++s)
            if (ok[s])
                atomicOr(bm + ids[s] * kWords, 1u << (t & 31));
    }
    __syncthreads();
    for (int c = t; c < cells; c += 1024) {
        int n = 0;
#pragma unroll
        for (int w = 0; w < kWords; ++w)
            n += __popc(s_bm[c * kWords + w]);
        s_cnt[c] = n;
    }
    __syncthreads();
    scan_block(T, k, E, D, my_rank, d, fp8, C, nchunks, s_cnt, invalid, o);
    // in-chunk position of (t, s): earlier tokens of the chunk routed to
    // the same expert
    if (t >= T)
        return;
    const uint32_t bit = 1u << (t & 31);
    const int wi = (t % kChunk) >> 5;
    const uint32_t *bm = s_bm + (size_t)(t / kChunk) * E * kWords;
#pragma unroll
    for (int s = 0; s < KM; ++s) {
        if (s >= k)
            break;
        int p = -1;
        if (ok[s]) {
            const uint32_t *m = bm + ids[s] * kWords;
            p = __popc(m[wi] & (bit - 1u));
            for (int w = 0; w < wi; ++w)
                p += __popc(m[w]);
        }
        pos_in_chunk[(size_t)t * k + s] = p;
    }
}

// a. Assignment a = t*k + s of expert e goes to by_expert[all_offset[e] + its
//    token-order position]: each expert's segment lists its assignments in
//    ascending token order.
__global__ __launch_bounds__(256) void group_by_expert_kernel(
    const int32_t *__restrict__ topk_idx, const int32_t *__restrict__ pos_in_chunk,
    const int32_t *__restrict__ chunk_base, const int32_t *__restrict__ all_offset, int T,
    int k, int E, int32_t *__restrict__ by_expert)
{
    const long long a = (long long)blockIdx.x * 256 + threadIdx.x;
    if (a >= (long long)T * k)
        return;
    const int p = pos_in_chunk[a];
    if (p < 0) // invalid entry
        return;
    const int t = (int)(a / k);
    const int e = topk_idx[a];
    by_expert[all_offset[e] + chunk_base[(size_t)(t / kChunk) * E + e] + p] = (int32_t)a;
}

// Order key of a gate value under drop policy 1: the fp32 bits mapped to an
// unsigned integer with the same order (-0 taken as +0).
__device__ __forceinline__ uint32_t gate_key(float g)
{
    uint32_t b = __float_as_uint(g);
    if (b == 0x80000000u)
        b = 0u;
    return (b & 0x80000000u) ? ~b : (b | 0x80000000u);
}

constexpr int kSelCache = 16384; // gate keys an expert keeps in LDS (more: re-read)

// b. One workgroup of 1024 threads per expert.  If the expert holds n > C
// assignments, a most-significant-digit radix select (four 8-bit digits)
// finds the gate key g* of the C-th largest gate and how many of the
// assignments with gate exactly g* still fit (m >= 1).  Because the list is
// in token order, the tie rule (equal gates: lower token first) keeps the
// first m of those in list order.  The kept ones are then numbered in list
// order: position = #(g > g*) before + min(#(g = g*) before, m), from one
// block scan of the two packed counts.
__global__ __launch_bounds__(1024) void gate_select_kernel(
    const int32_t *__restrict__ by_expert, const int32_t *__restrict__ all_offset,
    const int32_t *__restrict__ expert_count, const float *__restrict__ topk_w,
    long long C, int32_t *__restrict__ slot)
{
    __shared__ uint32_t s_key[kSelCache];
    __shared__ uint32_t hist[256];
    __shared__ uint32_t s_wave[kMaxExperts / 64];
    __shared__ uint32_t s_prefix;
    __shared__ int s_want;
    const int e = blockIdx.x, tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int n = expert_count[e];
    const int32_t *list = by_expert + all_offset[e];
    if (n <= C) { // everything fits: the token-order positions stand
        for (int i = tid; i < n; i += 1024)
            slot[list[i]] = i;
        return;
    }
    const bool cached = n <= kSelCache;
    if (cached)
        for (int i = tid; i < n; i += 1024)
            s_key[i] = gate_key(topk_w[list[i]]);
    auto key_of = [&](int i) { return cached ? s_key[i] : gate_key(topk_w[list[i]]); };
    uint32_t prefix = 0, mask = 0;
    int want = (int)C; // rank, among keys matching prefix, of the wanted key
    for (int shift = 24; shift >= 0; shift -= 8) {
        if (tid < 256)
            hist[tid] = 0u;
        __syncthreads();
        for (int i = tid; i < n; i += 1024) {
            const uint32_t key = key_of(i);
            if ((key & mask) == prefix)
                atomicAdd(&hist[(key >> shift) & 255u], 1u);
        }
        __syncthreads();
        if (wave == 0) {
            // lane l holds digits 255-4l .. 252-4l (largest first)
            uint32_t c[4];
            int tot = 0;
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                c[j] = hist[255 - (4 * lane + j)];
                tot += (int)c[j];
            }
            int incl = tot;
#pragma unroll
            for (int off = 1; off < 64; off <<= 1) {
                const int o = __shfl_up(incl, off, 64);
                if (lane >= off)
                    incl += o;
            }
            const unsigned long long hit = __ballot(incl >= want);
            if (lane == __ffsll((long long)hit) - 1) {
                int above = incl - tot;
                int digit = 0;
#pragma unroll
                for (int j = 0; j < 4; ++j) {
                    if (above + (int)c[j] >= want) {
                        digit = 255 - (4 * lane + j);
                        break;
                    }
                    above += (int)c[j];
                }
                s_want = want - above;
                s_prefix = prefix | ((uint32_t)digit << shift);
            }
        }
        __syncthreads();
        want = s_want;
        prefix = s_prefix;
        mask |= 255u << shift;
    }
    const uint32_t thr = prefix; // g*; `want` of the keys equal to it are kept
    int gt_carry = 0, eq_carry = 0;
    for (int base = 0; base < n; base += 1024) {
        const int i = base + tid;
        const uint32_t key = i < n ? key_of(i) : 0u;
        const uint32_t gt = (i < n && key > thr) ? 1u : 0u;
        const uint32_t eq = (i < n && key == thr) ? 1u : 0u;
        const uint32_t v = gt | (eq << 16); // per-tile counts stay below 2^16
        uint32_t incl = v;
#pragma unroll
        for (int off = 1; off < 64; off <<= 1) {
            const uint32_t o = __shfl_up(incl, off, 64);
            if (lane >= off)
                incl += o;
        }
        if (lane == 63)
            s_wave[wave] = incl;
        __syncthreads();
        uint32_t before = 0, total = 0;
        for (int w = 0; w < kMaxExperts / 64; ++w) {
            before += w < wave ? s_wave[w] : 0u;
            total += s_wave[w];
        }
        const uint32_t ex = before + incl - v;
        const int gt_before = gt_carry + (int)(ex & 0xffffu);
        const int eq_before = eq_carry + (int)(ex >> 16);
        if (i < n) {
            const bool keep = gt || (eq && eq_before < want);
            slot[list[i]] = keep ? gt_before + min(eq_before, want) : -1;
        }
        gt_carry += (int)(total & 0xffffu);
        eq_carry += (int)(total >> 16);
        __syncthreads();
    }
}

constexpr int kSlotGroup = 8; // slots resolved per pass over a token row

// One token row of d bf16 as E4M3 codes with one fp32 scale (dispatch
// payload of FP8 mode): s = amax/448 (1 for an all-zero row), code of
// x/s (IEEE fp32 quotient).  The wave reads the row twice (the second time
// from L2): once for amax, once to encode.
__device__ __forceinline__ float row_scale_e4m3(const uint4 *src, int nvec, int lane)
{
    float amax = 0.f;
    for (int c = lane; c < nvec; c += 64) {
        const uint4 v = src[c];
        const uint32_t p[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
        for (int q = 0; q < 4; ++q)
            amax = fmaxf(amax, fmaxf(fabsf(bf16_to_f32(p[q] & 0xffffu)),
                                     fabsf(bf16_to_f32(p[q] >> 16))));
    }
#pragma unroll
    for (int off = 32; off > 0; off >>= 1)
        amax = fmaxf(amax, __shfl_xor(amax, off, 64));
    return amax > 0.f ? amax / 448.f : 1.f;
}

__device__ __forceinline__ uint2 encode8_e4m3(uint4 v, float sc)
{
    const uint32_t p[4] = {v.x, v.y, v.z, v.w};
    uint32_t w[2];
#pragma unroll
    for (int h = 0; h < 2; ++h) {
        const uint32_t a = p[2 * h], b = p[2 * h + 1];
        w[h] = e4m3_from_f32(bf16_to_f32(a & 0xffffu) / sc) |
               (e4m3_from_f32(bf16_to_f32(a >> 16) / sc) << 8) |
               (e4m3_from_f32(bf16_to_f32(b & 0xffffu) / sc) << 16) |
               (e4m3_from_f32(bf16_to_f32(b >> 16) / sc) << 24);
    }
    return make_uint2(w[0], w[1]);
}

// send_buf rows are d bf16 (FP8 = false) or d E4M3 codes with their scale in
// send_scale (FP8 = true).
template <bool FP8>
__global__ __launch_bounds__(256) void permute_kernel(
    const uint16_t *__restrict__ x, const int32_t *__restrict__ topk_idx,
    int32_t *__restrict__ slot, const int32_t *__restrict__ chunk_base,
    const int32_t *__restrict__ expert_offset, const int32_t *__restrict__ expert_kept,
    void *__restrict__ send_buf_v, float *__restrict__ send_scale, int T, int d, int k, int E,
    long long C, int tok_blocks, int pad_parts, int pos_final, int W)
{
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const int nvec = d / 8;                    // 16-byte pieces of an x row
    const size_t row_bytes = (size_t)d * (FP8 ? 1 : 2);
    char *send_buf = reinterpret_cast<char *>(send_buf_v);
    if ((int)blockIdx.x < tok_blocks) {
        // W waves per token (1, 2 or 4: a token's waves share a workgroup);
        // wave h copies the contiguous pieces [h n / W, (h+1) n / W)
        const int gw = blockIdx.x * 4 + wave;
        const int h = gw % W;
        const bool valid = gw / W < T;
        if (!valid && W == 1)
            return; // (W > 1: every wave reaches the workgroup barriers)
        const int t = valid ? gw / W : T - 1; // a wave past T mirrors the last token, writes nothing
        const int c_lo = (int)((long long)h * nvec / W), c_hi = (int)((long long)(h + 1) * nvec / W);
        const int32_t *row = topk_idx + (size_t)t * k;
        const int32_t *base = chunk_base + (size_t)(t / kChunk) * E;
        const uint4 *src = reinterpret_cast<const uint4 *>(x + (size_t)t * d);
        float sc = 1.f;
        if constexpr (FP8)
            sc = row_scale_e4m3(src, nvec, lane);
        for (int s0 = 0; s0 < k; s0 += kSlotGroup) {
            // The slots are wave-uniform: resolve them in scalar registers,
            // in two rounds of loads (positions and experts, then the chunk
            // bases and expert offsets) with every load of a round in flight
            // together; an entry with no position reads expert 0's values
            // and ignores them.
            int pq[kSlotGroup], eq[kSlotGroup], dst[kSlotGroup];
#pragma unroll
            for (int q = 0; q < kSlotGroup; ++q) {
                const int s = s0 + q;
                // in-chunk position (in-expert position if pos_final), or -1
                pq[q] = s < k ? __builtin_amdgcn_readfirstlane(slot[(size_t)t * k + s]) : -1;
                eq[q] = s < k ? __builtin_amdgcn_readfirstlane(row[s]) : 0;
            }
#pragma unroll
            for (int q = 0; q < kSlotGroup; ++q) {
                const int e = pq[q] >= 0 ? eq[q] : 0; // a valid entry's expert is in [0, E)
                const long long pos =
                    pos_final ? pq[q] : (long long)__builtin_amdgcn_readfirstlane(base[e]) + pq[q];
                const int off = __builtin_amdgcn_readfirstlane(expert_offset[e]);
                dst[q] = (pq[q] >= 0 && (C < 0 || pos < C)) ? off + (int)pos : -1;
            }
            // every lane (and every wave of the token) has read the
            // positions before lane 0 of wave 0 overwrites them
            __builtin_amdgcn_wave_barrier();
            if (W > 1)
                __syncthreads();
            if (!valid)
                continue;
            if (h == 0 && lane < kSlotGroup && s0 + lane < k) {
                int v = dst[0];
#pragma unroll
                for (int q = 1; q < kSlotGroup; ++q)
                    v = (lane == q) ? dst[q] : v;
                slot[(size_t)t * k + s0 + lane] = v;
                if constexpr (FP8)
                    if (v >= 0)
                        send_scale[v] = sc;
            }
            // four row pieces in flight per lane before their stores; the
            // stores are non-temporal (the rows are read by the GEMM only)
            for (int c0 = c_lo + lane; c0 < c_hi; c0 += 256) {
                uint4 v[4];
#pragma unroll
                for (int u = 0; u < 4; ++u)
                    v[u] = (c0 + 64 * u < c_hi) ? src[c0 + 64 * u] : make_uint4(0, 0, 0, 0);
                if constexpr (FP8) {
                    uint2 q8[4];
#pragma unroll
                    for (int u = 0; u < 4; ++u)
                        q8[u] = encode8_e4m3(v[u], sc);
#pragma unroll
                    for (int q = 0; q < kSlotGroup; ++q) {
                        if (dst[q] < 0)
                            continue;
                        uint2 *out = reinterpret_cast<uint2 *>(send_buf + (size_t)dst[q] * row_bytes);
#pragma unroll
                        for (int u = 0; u < 4; ++u)
                            if (c0 + 64 * u < c_hi)
                                store_nt(out + c0 + 64 * u, q8[u]);
                    }
                } else {
#pragma unroll
                    for (int q = 0; q < kSlotGroup; ++q) {
                        if (dst[q] < 0)
                            continue;
                        uint4 *out = reinterpret_cast<uint4 *>(send_buf + (size_t)dst[q] * row_bytes);
#pragma unroll
                        for (int u = 0; u < 4; ++u)
                            if (c0 + 64 * u < c_hi)
                                store_nt(out + c0 + 64 * u, v[u]);
                    }
                }
            }
        }
        return;
    }
    // pad rows (capacity mode) and the dropless tail: zero bytes (E4M3 code
    // 0 is +0), scale 0
    const int nz = (int)(row_bytes / 16);
    const uint4 z = make_uint4(0, 0, 0, 0);
    long long r_lo, r_hi, r_step;
    int r_off;
    const int b = blockIdx.x - tok_blocks;
    if (C < 0) {
        // dropless: rows [offset[E], T*k) hold no token (they exist only when
        // entries were invalid); zero them so the whole buffer is defined
        r_lo = expert_offset[E];
        r_hi = (long long)T * k;
        r_off = b * 4 + wave;
        r_step = (long long)pad_parts * 4;
    } else {
        // the pad rows [e*C + kept_e, (e+1)*C) of capacity mode
        const int e = b / pad_parts, part = b % pad_parts;
        const long long per = (C + pad_parts - 1) / pad_parts;
        const long long lo_pad = (long long)e * C + expert_kept[e];
        r_lo = max((long long)e * C + part * per, lo_pad);
        r_hi = min((long long)e * C + (part + 1) * per, (long long)(e + 1) * C);
        r_off = wave;
        r_step = 4;
    }
    for (long long r = r_lo + r_off; r < r_hi; r += r_step) {
        uint4 *dstp = reinterpret_cast<uint4 *>(send_buf + (size_t)r * row_bytes);
        for (int c = lane; c < nz; c += 64)
            dstp[c] = z;
        if constexpr (FP8)
            if (lane == 0)
                send_scale[r] = 0.f;
    }
}

// Diagnostic: out[r, i] = bf16(E4M3 value of codes[r, i] * scales[r]), the
// decode the expert GEMM uses; exact when the scale is a power of two.
__global__ __launch_bounds__(256) void fp8_rows_to_bf16_kernel(const uint8_t *__restrict__ codes,
                                                               const float *__restrict__ scales,
                                                               long long rows, int d,
                                                               uint16_t *__restrict__ out)
{
    const long long q = (long long)blockIdx.x * 256 + threadIdx.x; // 4 codes each
    if (q >= rows * (d / 4))
        return;
    const long long r = q / (d / 4);
    const uint32_t w = reinterpret_cast<const uint32_t *>(codes)[q];
    const uint2 b = e4m3x4_to_bf16x4(w);
    const float sc = scales ? scales[r] : 1.f;
    const uint32_t v[4] = {b.x & 0xffffu, b.x >> 16, b.y & 0xffffu, b.y >> 16};
    uint16_t *o = out + q * 4;
#pragma unroll
    for (int i = 0; i < 4; ++i)
        o[i] = (uint16_t)f32_to_bf16_rne(bf16_to_f32(v[i]) * sc);
}

} // namespace

hipError_t launch_dispatch(const Dims &dm, const uint16_t *x, const int32_t *topk_idx,
                           const float *topk_w, void *send_buf, float *send_scale, int32_t *slot,
                           int32_t *expert_count, int32_t *expert_kept, int32_t *expert_offset,
                           int32_t *rank_rows, moe_stats *stats, char *ws, const Workspace &wl,
                           hipStream_t st)
{
    int32_t *chunk_counts = reinterpret_cast<int32_t *>(ws + wl.chunk_counts);
    int32_t *chunk_base = reinterpret_cast<int32_t *>(ws + wl.chunk_base);
    int32_t *chunk_invalid = reinterpret_cast<int32_t *>(ws + wl.chunk_invalid);
    const bool by_gate = dm.drop_policy == 1 && dm.capacity >= 0;
    int32_t *all_offset = by_gate ? reinterpret_cast<int32_t *>(ws + wl.all_offset) : nullptr;
    int32_t *by_expert = reinterpret_cast<int32_t *>(ws + wl.by_expert);
    const ScanOut so{chunk_base, expert_count, expert_kept, expert_offset, rank_rows, stats,
                      all_offset};
    // Count and scan in one workgroup only up to four chunks: one CU then
    // does every chunk's bitmap work, which costs more than the second
    // launch once there are many chunks (DeepSeek-V3 prefill, 16 chunks:
    // 60.8 us against 9.0 + 7.6 us for the two kernels).
    const bool fused = dm.T <= 1024 && dm.k <= 8 && (long long)dm.nchunks * dm.E <= kFusedCells;
    if (fused) {
#define MOE_COUNT_SCAN(KM)                                                                   \
    count_scan_kernel<KM><<<1, 1024, 0, st>>>(topk_idx, dm.T, dm.k, dm.E, dm.D, dm.my_rank,   \
                                              dm.d, dm.fp8, (long long)dm.capacity,           \
                                              dm.nchunks, slot, so)
        if (dm.k <= 2)
            MOE_COUNT_SCAN(2);
        else if (dm.k <= 4)
            MOE_COUNT_SCAN(4);
        else
            MOE_COUNT_SCAN(8);
#undef MOE_COUNT_SCAN
    } else {
        const size_t lds = (size_t)dm.E * kWords * sizeof(uint32_t);
#define MOE_COUNT(KM)                                                                        \
    count_kernel<KM><<<dm.nchunks, kChunk, lds, st>>>(topk_idx, dm.T, dm.k, dm.E, slot,      \
                                                      chunk_counts, chunk_invalid)
        if (dm.k <= 2)
            MOE_COUNT(2);
        else if (dm.k <= 4)
            MOE_COUNT(4);
        else if (dm.k <= 8)
            MOE_COUNT(8);
        else if (dm.k <= 16)
            MOE_COUNT(16);
        else
            MOE_COUNT(0);
#undef MOE_COUNT
        scan_kernel<<<1, kMaxExperts, 0, st>>>(dm.T, dm.k, dm.E, dm.D, dm.my_rank, dm.d, dm.fp8,
                                               (long long)dm.capacity, dm.nchunks, chunk_counts,
                                               chunk_invalid, so);
    }
    if (by_gate && dm.T > 0) {
        const long long a = (long long)dm.T * dm.k;
        group_by_expert_kernel<<<(unsigned)((a + 255) / 256), 256, 0, st>>>(
            topk_idx, slot, chunk_base, all_offset, dm.T, dm.k, dm.E, by_expert);
        gate_select_kernel<<<dm.E, 1024, 0, st>>>(by_expert, all_offset, expert_count, topk_w,
                                                   (long long)dm.capacity, slot);
    }
    // waves per token: one when the tokens give the launch 4096 wavefronts
    // (16 per CU), else two or four (DeepSeek-V3 decode: 64 tokens)
    const int pw = dm.T >= 4096 ? 1 : dm.T >= 2048 ? 2 : 4;
    const int tok_blocks = (int)(((long long)dm.T * pw + 3) / 4);
    int pad_parts = 0;
    long long pad_blocks = 0;
    if (dm.capacity > 0) {
        // split each expert's C rows so that the pad zeroing spreads over ~1024 workgroups
        pad_parts = (int)std::max<long long>(1, std::min<long long>(dm.capacity, 1024 / dm.E));
        pad_blocks = (long long)dm.E * pad_parts;
    } else if (dm.capacity < 0 && dm.T > 0) {
        // dropless tail: a few grid-stride workgroups (idle unless entries were invalid)
        pad_parts = 16;
        pad_blocks = pad_parts;
    }
    const long long blocks = (long long)tok_blocks + pad_blocks;
    if (blocks > 0) {
        if (dm.fp8)
            permute_kernel<true><<<(unsigned)blocks, 256, 0, st>>>(
                x, topk_idx, slot, chunk_base, expert_offset, expert_kept, send_buf, send_scale,
                dm.T, dm.d, dm.k, dm.E, (long long)dm.capacity, tok_blocks, pad_parts,
                by_gate ? 1 : 0, pw);
        else
            permute_kernel<false><<<(unsigned)blocks, 256, 0, st>>>(
                x, topk_idx, slot, chunk_base, expert_offset, expert_kept, send_buf, nullptr,
                dm.T, dm.d, dm.k, dm.E, (long long)dm.capacity, tok_blocks, pad_parts,
                by_gate ? 1 : 0, pw);
    }
    return hipGetLastError();
}

hipError_t launch_fp8_rows_to_bf16(const uint8_t *codes, const float *scales, long long rows,
                                   int d, uint16_t *out, hipStream_t st)
{
    const long long quads = rows * (d / 4);
    if (quads == 0)
        return hipSuccess;
    fp8_rows_to_bf16_kernel<<<(unsigned)((quads + 255) / 256), 256, 0, st>>>(codes, scales,
                                                                             rows, d, out);
    return hipGetLastError();
}

} // namespace moe
