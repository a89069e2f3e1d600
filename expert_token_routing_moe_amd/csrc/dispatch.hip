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
//  3. permute: a wavefront per token turns positions into slots, reads the
//     token row once and writes it to each kept slot with 16-byte stores;
//     extra workgroups zero the pad rows of capacity mode.
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
    for (int w = i; w < E * kWords; w += kChunk)
        bm[w] = 0u;
    if (i == 0)
        s_invalid = 0;
    __syncthreads();
    const int32_t *row = topk_idx + (size_t)t * k;
    const uint32_t bit = 1u << (i & 31);
    if (t < T) {
        for (int s = 0; s < k; ++s)
            if (entry_valid(row, s, E))
                atomicOr(&bm[row[s] * kWords + (i >> 5)], bit);
    }
    __syncthreads();
    if (t < T) {
        int invalid = 0;
        for (int s = 0; s < k; ++s) {
            int32_t p = -1;
            if (entry_valid(row, s, E)) {
                const uint32_t *m = bm + row[s] * kWords;
                p = __popc(m[i >> 5] & (bit - 1u));
                for (int w = 0; w < (i >> 5); ++w)
                    p += __popc(m[w]);
            } else {
                ++invalid;
            }
            pos_in_chunk[(size_t)t * k + s] = p;
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

// Single workgroup of 1024 threads: thread e owns expert e.
__global__ __launch_bounds__(kMaxExperts) void scan_kernel(
    int T, int k, int E, int D, int my_rank, int d, long long C, int nchunks,
    const int32_t *__restrict__ chunk_counts, int32_t *__restrict__ chunk_base,
    const int32_t *__restrict__ chunk_invalid, int32_t *__restrict__ expert_count,
    int32_t *__restrict__ expert_kept, int32_t *__restrict__ expert_offset,
    int32_t *__restrict__ rank_rows, moe_stats *__restrict__ stats)
{
    __shared__ int32_t s_n[kMaxExperts], s_kept[kMaxExperts];
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
        for (int c = 0; c < nchunks; ++c) {
            chunk_base[(size_t)c * E + e] = n;
            n += chunk_counts[(size_t)c * E + e];
        }
        kept = (C < 0 || n < C) ? n : (int)C;
        expert_count[e] = n;
        expert_kept[e] = kept;
    }
    s_n[e] = n;
    s_kept[e] = kept;
    // exclusive scan of n over experts (dropless offsets): wave scan + wave totals
    int incl = n;
#pragma unroll
    for (int off = 1; off < 64; off <<= 1) {
        const int o = __shfl_up(incl, off, 64);
        if (lane >= off)
            incl += o;
    }
    if (lane == 63)
        s_wave_sum[wave] = incl;
    __syncthreads();
    int wave_base = 0;
    for (int w = 0; w < wave; ++w)
        wave_base += s_wave_sum[w];
    const int excl = wave_base + incl - n;
    if (e < E)
        expert_offset[e] = (C < 0) ? excl : (int)((long long)e * C);
    if (e == E - 1)
        expert_offset[E] = (C < 0) ? excl + n : (int)((long long)E * C);
    // reductions
    if (e < E) {
        atomicAdd(&s_kept_total, kept);
        atomicMax(&s_max, n);
    }
    for (int c = e; c < nchunks; c += kMaxExperts)
        atomicAdd(&s_invalid, chunk_invalid[c]);
    const int epr = E / D;
    for (int r = e; r < D; r += kMaxExperts) {
        int rows = 0;
        for (int q = r * epr; q < (r + 1) * epr; ++q)
            rows += s_kept[q];
        rank_rows[r] = rows;
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
        st.dispatch_bytes = kt * d * 2;
        st.dispatch_wire_bytes = (C < 0) ? kt * d * 2 : send_rows * d * 2;
        st.dispatch_remote_bytes = (long long)s_remote * d * 2;
        st.combine_bytes = kt * d * 2;
        st.max_expert_count = s_max;
        st.invalid_index = s_invalid;
        *stats = st;
    }
}

constexpr int kSlotGroup = 8; // slots resolved per pass over a token row

__global__ __launch_bounds__(256) void permute_kernel(
    const uint16_t *__restrict__ x, const int32_t *__restrict__ topk_idx,
    int32_t *__restrict__ slot, const int32_t *__restrict__ chunk_base,
    const int32_t *__restrict__ expert_offset, const int32_t *__restrict__ expert_kept,
    uint16_t *__restrict__ send_buf, int T, int d, int k, int E, long long C, int tok_blocks,
    int pad_parts)
{
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const int nvec = d / 8; // 16-byte vectors per row
    if ((int)blockIdx.x < tok_blocks) {
        const int t = blockIdx.x * 4 + wave;
        if (t >= T)
            return;
        const int32_t *row = topk_idx + (size_t)t * k;
        const int32_t *base = chunk_base + (size_t)(t / kChunk) * E;
        const uint4 *src = reinterpret_cast<const uint4 *>(x + (size_t)t * d);
        for (int s0 = 0; s0 < k; s0 += kSlotGroup) {
            // the slots are wave-uniform: resolve them in scalar registers
            int dst[kSlotGroup];
#pragma unroll
            for (int q = 0; q < kSlotGroup; ++q) {
                const int s = s0 + q;
                int sl = -1;
                if (s < k) {
                    // in-chunk position, or -1
                    const int p = __builtin_amdgcn_readfirstlane(slot[(size_t)t * k + s]);
                    if (p >= 0) {
                        const int e = __builtin_amdgcn_readfirstlane(row[s]);
                        const long long pos =
                            (long long)__builtin_amdgcn_readfirstlane(base[e]) + p;
                        if (C < 0 || pos < C)
                            sl = __builtin_amdgcn_readfirstlane(expert_offset[e]) + (int)pos;
                    }
                }
                dst[q] = sl;
            }
            // every lane has read the positions before lane 0 overwrites them
            __builtin_amdgcn_wave_barrier();
            if (lane < kSlotGroup && s0 + lane < k) {
                int v = dst[0];
#pragma unroll
                for (int q = 1; q < kSlotGroup; ++q)
                    v = (lane == q) ? dst[q] : v;
                slot[(size_t)t * k + s0 + lane] = v;
            }
            // four row pieces in flight per lane before their stores
            for (int c0 = lane; c0 < nvec; c0 += 256) {
                uint4 v[4];
#pragma unroll
                for (int u = 0; u < 4; ++u)
                    v[u] = (c0 + 64 * u < nvec) ? src[c0 + 64 * u] : make_uint4(0, 0, 0, 0);
#pragma unroll
                for (int q = 0; q < kSlotGroup; ++q) {
                    if (dst[q] < 0)
                        continue;
                    uint4 *out = reinterpret_cast<uint4 *>(send_buf + (size_t)dst[q] * d);
#pragma unroll
                    for (int u = 0; u < 4; ++u)
                        if (c0 + 64 * u < nvec)
                            out[c0 + 64 * u] = v[u];
                }
            }
        }
    } else if (C < 0) {
        // dropless: rows [offset[E], T*k) hold no token (they exist only when
        // entries were invalid); zero them so the whole buffer is defined
        const long long lo = expert_offset[E], hi = (long long)T * k;
        const int b = blockIdx.x - tok_blocks;
        const uint4 z = make_uint4(0, 0, 0, 0);
        for (long long r = lo + b * 4 + wave; r < hi; r += (long long)pad_parts * 4) {
            uint4 *dstp = reinterpret_cast<uint4 *>(send_buf + (size_t)r * d);
            for (int c = lane; c < nvec; c += 64)
                dstp[c] = z;
        }
    } else {
        // zero the pad rows [e*C + kept_e, (e+1)*C) of capacity mode
        const int b = blockIdx.x - tok_blocks;
        const int e = b / pad_parts, part = b % pad_parts;
        const long long per = (C + pad_parts - 1) / pad_parts;
        const long long lo_pad = (long long)e * C + expert_kept[e];
        const long long r_lo = max((long long)e * C + part * per, lo_pad);
        const long long r_hi = min((long long)e * C + (part + 1) * per, (long long)(e + 1) * C);
        const uint4 z = make_uint4(0, 0, 0, 0);
        for (long long r = r_lo + wave; r < r_hi; r += 4) {
            uint4 *dstp = reinterpret_cast<uint4 *>(send_buf + (size_t)r * d);
            for (int c = lane; c < nvec; c += 64)
                dstp[c] = z;
        }
    }
}

} // namespace

hipError_t launch_dispatch(const Dims &dm, const uint16_t *x, const int32_t *topk_idx,
                           uint16_t *send_buf, int32_t *slot, int32_t *expert_count,
                           int32_t *expert_kept, int32_t *expert_offset, int32_t *rank_rows,
                           moe_stats *stats, char *ws, const Workspace &wl, hipStream_t st)
{
    int32_t *chunk_counts = reinterpret_cast<int32_t *>(ws + wl.chunk_counts);
    int32_t *chunk_base = reinterpret_cast<int32_t *>(ws + wl.chunk_base);
    int32_t *chunk_invalid = reinterpret_cast<int32_t *>(ws + wl.chunk_invalid);
    if (dm.nchunks > 0) {
        const size_t lds = (size_t)dm.E * kWords * sizeof(uint32_t);
        count_kernel<<<dm.nchunks, kChunk, lds, st>>>(topk_idx, dm.T, dm.k, dm.E, slot,
                                                       chunk_counts, chunk_invalid);
    }
    scan_kernel<<<1, kMaxExperts, 0, st>>>(dm.T, dm.k, dm.E, dm.D, dm.my_rank, dm.d,
                                           (long long)dm.capacity, dm.nchunks, chunk_counts,
                                           chunk_base, chunk_invalid, expert_count, expert_kept,
                                           expert_offset, rank_rows, stats);
    const int tok_blocks = (dm.T + 3) / 4;
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
    if (blocks > 0)
        permute_kernel<<<(unsigned)blocks, 256, 0, st>>>(
            x, topk_idx, slot, chunk_base, expert_offset, expert_kept, send_buf, dm.T, dm.d,
            dm.k, dm.E, (long long)dm.capacity, tok_blocks, pad_parts);
    return hipGetLastError();
}

} // namespace moe
