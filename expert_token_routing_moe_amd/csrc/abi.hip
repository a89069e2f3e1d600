// C ABI of the library (declared in include/moe.h): host-side validation,
// workspace carving and stream-ordered launch sequencing.  No allocation, no
// host synchronisation, no state kept between calls.
#include <math.h>

#include <algorithm>
#include <mutex>

#include "moe_internal.hpp"

#define MOE_EXPORT extern "C" __attribute__((visibility("default")))

namespace moe {

static size_t align_up(size_t v) { return (v + 255) & ~(size_t)255; }

Workspace workspace_layout(const Dims &dm)
{
    Workspace w{};
    size_t off = 0;
    auto take = [&](size_t bytes) {
        const size_t at = off;
        off = align_up(off + bytes);
        return at;
    };
    w.logits = take(router_partials(dm.T, dm.E, dm.d) ? (size_t)router_ksplit(dm.T, dm.E, dm.d) *
                                                            dm.T * router_epad(dm.E) * sizeof(float)
                                                      : 0);
    w.wg_pad = take(router_ldw(dm.E) != dm.E ? (size_t)dm.d * router_ldw(dm.E) * sizeof(uint16_t)
                                             : 0);
    w.chunk_counts = take((size_t)dm.nchunks * dm.E * sizeof(int32_t));
    w.chunk_base = take((size_t)dm.nchunks * dm.E * sizeof(int32_t));
    w.chunk_invalid = take((size_t)dm.nchunks * sizeof(int32_t));
    const bool by_gate = dm.drop_policy == 1 && dm.capacity >= 0;
    w.all_offset = take(by_gate ? (size_t)dm.E * sizeof(int32_t) : 0);
    w.by_expert = take(by_gate ? (size_t)dm.T * dm.k * sizeof(int32_t) : 0);
    w.h = take((size_t)dm.send_rows * dm.H * sizeof(uint16_t));
    w.a_wide = take(dm.fp8_widen ? (size_t)dm.send_rows * dm.d * sizeof(uint16_t) : 0);
    w.shared_rows = take(dm.shared_H > 0 ? 4 * sizeof(int32_t) : 0);
    w.shared_h = take((size_t)(dm.shared_H > 0 ? dm.T : 0) * dm.shared_H * sizeof(uint16_t));
    w.total = std::max<size_t>(off, 256);
    return w;
}

// Validates the shape and derives the per-call facts; MOE_OK or an error.
static int make_dims(const moe_shape *s, Dims *dm)
{
    if (!s)
        return MOE_EINVAL;
    if (s->T < 0 || s->d <= 0 || s->E <= 0 || s->k <= 0 || s->H <= 0 || s->D <= 0)
        return MOE_EINVAL;
    if (s->k > s->E || s->E % s->D != 0 || s->my_rank < 0 || s->my_rank >= s->D)
        return MOE_EINVAL;
    const double cf = s->capacity_factor;
    if (isnan(cf) || cf <= 0.0)
        return MOE_EINVAL;
    if (s->d % 8 != 0)
        return MOE_EINVAL;
    if (s->drop_policy != 0 && s->drop_policy != 1)
        return MOE_EINVAL;
    if (s->min_capacity < 0)
        return MOE_EINVAL;
    if (s->dispatch_fp8 != 0 && s->dispatch_fp8 != 1)
        return MOE_EINVAL;
    // group-limited routing: G equal groups, at most M per token, k of them
    // must be reachable
    if (s->n_groups < 0 || s->shared_H < 0)
        return MOE_EINVAL;
    const bool grouped = s->n_groups > 1 && s->group_limit < s->n_groups;
    if (s->n_groups > 1 && (s->E % s->n_groups != 0 || s->group_limit < 1))
        return MOE_EINVAL;
    if (grouped && (long long)s->group_limit * (s->E / s->n_groups) < s->k)
        return MOE_EINVAL;
    if (s->shared_H % 64 != 0)
        return MOE_EUNSUPPORTED;
    if (s->d % 64 != 0 || s->H % 64 != 0 || s->E > kMaxExperts)
        return MOE_EUNSUPPORTED;
    const long long assignments = (long long)s->T * s->k;
    if (assignments > INT32_MAX)
        return MOE_EUNSUPPORTED;
    long long C = -1, send_rows = assignments;
    if (!isinf(cf)) {
        // C = ceil(cf * T * k / E), evaluated left to right in double, then
        // raised to the minimum capacity
        const double c = ceil(cf * (double)s->T * (double)s->k / (double)s->E);
        if (c > (double)INT32_MAX)
            return MOE_EUNSUPPORTED;
        C = std::max<long long>((long long)c, s->min_capacity);
        send_rows = (long long)s->E * C;
    }
    if (send_rows > INT32_MAX)
        return MOE_EUNSUPPORTED;
    // grouped-GEMM grids: (row tiles + E) * N tiles must fit a 1-D grid
    const long long mtiles = (send_rows + 127) / 128 + s->E;
    if (mtiles * (s->H / 64) > INT32_MAX / 2 || mtiles * (s->d / 64) > INT32_MAX / 2)
        return MOE_EUNSUPPORTED;
    dm->T = s->T;
    dm->d = s->d;
    dm->E = s->E;
    dm->k = s->k;
    dm->H = s->H;
    dm->D = s->D;
    dm->my_rank = s->my_rank;
    dm->drop_policy = s->drop_policy;
    dm->fp8 = s->dispatch_fp8;
    dm->n_groups = grouped ? s->n_groups : 1;
    dm->group_limit = grouped ? s->group_limit : 1;
    dm->shared_H = s->shared_H;
    dm->capacity = C;
    dm->send_rows = send_rows;
    // rows an expert is expected to hold: C, or the mean T*k/E when dropless
    const int64_t per_expert =
        C >= 0 ? C : ((int64_t)s->T * s->k + s->E - 1) / s->E;
    dm->mfma_bound = per_expert >= kMfmaBoundRows;
    dm->fp8_widen = s->dispatch_fp8 == 1 && dm->mfma_bound;
    dm->nchunks = (s->T + kChunk - 1) / kChunk;
    return MOE_OK;
}

// A required pointer may be NULL only when its tensor has no elements.
static bool bad_ptr(const void *p, long long elems = 1)
{
    return (p == nullptr && elems > 0) || ((uintptr_t)p & 15u) != 0;
}
static bool bad_opt_ptr(const void *p) { return p != nullptr && ((uintptr_t)p & 15u) != 0; }

static int check_ws(const Dims &dm, const void *ws, size_t ws_bytes, Workspace *wl)
{
    *wl = workspace_layout(dm);
    if (ws == nullptr || ((uintptr_t)ws & 255u) != 0 || ws_bytes < wl->total)
        return MOE_EWORKSPACE;
    return MOE_OK;
}

static int hip_status(hipError_t e) { return e == hipSuccess ? MOE_OK : MOE_EHIP; }

// The dispatch's own regions of a workspace, laid out from offset 0 (the
// scratch of moe_dispatch_noalloc).
static Workspace dispatch_layout(const Dims &dm)
{
    Workspace w{};
    size_t off = 0;
    auto take = [&](size_t bytes) {
        const size_t at = off;
        off = align_up(off + bytes);
        return at;
    };
    w.chunk_counts = take((size_t)dm.nchunks * dm.E * sizeof(int32_t));
    w.chunk_base = take((size_t)dm.nchunks * dm.E * sizeof(int32_t));
    w.chunk_invalid = take((size_t)dm.nchunks * sizeof(int32_t));
    const bool by_gate = dm.drop_policy == 1 && dm.capacity >= 0;
    w.all_offset = take(by_gate ? (size_t)dm.E * sizeof(int32_t) : 0);
    w.by_expert = take(by_gate ? (size_t)dm.T * dm.k * sizeof(int32_t) : 0);
    w.total = off;
    return w;
}

// Scratch of moe_dispatch_noalloc: one array per GPU, for the life of the
// process.  In host code `scratch` names a host-side stand-in, not the
// device array: its device address comes from hipGetSymbolAddress, taken
// once per device with that device current, and only that address is
// passed to kernels.
static __device__ __align__(256) char scratch[MOE_DISPATCH_SCRATCH_BYTES];
constexpr int kMaxDevices = 64;
static char *scratch_ptr[kMaxDevices];
static std::mutex scratch_mu;

// The current device's scratch address (looked up on its first use), or null
// with *err set.
static char *device_scratch(hipError_t *err)
{
    int dev = 0;
    *err = hipGetDevice(&dev);
    if (*err != hipSuccess)
        return nullptr;
    if (dev < 0 || dev >= kMaxDevices) {
        *err = hipErrorInvalidDevice;
        return nullptr;
    }
    std::lock_guard<std::mutex> lock(scratch_mu);
    if (!scratch_ptr[dev]) {
        void *p = nullptr;
        *err = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
        if (*err != hipSuccess)
            return nullptr;
        scratch_ptr[dev] = static_cast<char *>(p);
    }
    return scratch_ptr[dev];
}

} // namespace moe

using namespace moe;

MOE_EXPORT int moe_query(const moe_shape *shape, int64_t *send_rows, int64_t *capacity,
                         size_t *workspace_bytes)
{
    Dims dm;
    const int rc = make_dims(shape, &dm);
    if (rc != MOE_OK)
        return rc;
    if (send_rows)
        *send_rows = dm.send_rows;
    if (capacity)
        *capacity = dm.capacity;
    if (workspace_bytes)
        *workspace_bytes = workspace_layout(dm).total;
    return MOE_OK;
}

MOE_EXPORT int moe_route(const moe_shape *shape, const uint16_t *x, const uint16_t *w_gate,
                         const float *logit_bias, float *logits_out, int32_t *topk_idx,
                         float *topk_w, void *workspace, size_t workspace_bytes, void *stream)
{
    Dims dm;
    int rc = make_dims(shape, &dm);
    if (rc != MOE_OK)
        return rc;
    if (bad_ptr(x, dm.T) || bad_ptr(w_gate) || bad_ptr(topk_idx, dm.T) ||
        bad_ptr(topk_w, dm.T) || bad_opt_ptr(logit_bias) || bad_opt_ptr(logits_out))
        return MOE_EINVAL;
    Workspace wl;
    if ((rc = check_ws(dm, workspace, workspace_bytes, &wl)) != MOE_OK)
        return rc;
    return hip_status(launch_route(dm, x, w_gate, logit_bias, logits_out, topk_idx, topk_w,
                                   (char *)workspace, wl, static_cast<hipStream_t>(stream)));
}

MOE_EXPORT int moe_topk_from_logits(const moe_shape *shape, const float *logits,
                                    int32_t *topk_idx, float *topk_w, void *stream)
{
    Dims dm;
    const int rc = make_dims(shape, &dm);
    if (rc != MOE_OK)
        return rc;
    if (bad_ptr(logits, dm.T) || bad_ptr(topk_idx, dm.T) || bad_ptr(topk_w, dm.T))
        return MOE_EINVAL;
    return hip_status(launch_topk_softmax(dm, logits, topk_idx, topk_w,
                                          static_cast<hipStream_t>(stream)));
}

// The FP8 row scales: required (for a non-empty buffer) under FP8 dispatch.
static bool bad_scale(const Dims &dm, const float *send_scale)
{
    return dm.fp8 ? bad_ptr(send_scale, dm.send_rows) : bad_opt_ptr(send_scale);
}

MOE_EXPORT int moe_dispatch(const moe_shape *shape, const uint16_t *x, const int32_t *topk_idx,
                            const float *topk_w, void *send_buf, float *send_scale,
                            int32_t *slot, int32_t *expert_count, int32_t *expert_kept,
                            int32_t *expert_offset, int32_t *rank_rows, moe_stats *stats,
                            void *workspace, size_t workspace_bytes, void *stream)
{
    Dims dm;
    int rc = make_dims(shape, &dm);
    if (rc != MOE_OK)
        return rc;
    const bool need_w = dm.drop_policy == 1 && dm.capacity >= 0;
    if (need_w ? bad_ptr(topk_w, dm.T) : bad_opt_ptr(topk_w))
        return MOE_EINVAL;
    if (bad_scale(dm, send_scale))
        return MOE_EINVAL;
    if (bad_ptr(x, dm.T) || bad_ptr(topk_idx, dm.T) || bad_ptr(send_buf, dm.send_rows) ||
        bad_ptr(slot, dm.T) || bad_ptr(expert_count) || bad_ptr(expert_kept) ||
        bad_ptr(expert_offset) || bad_ptr(rank_rows) || bad_ptr(stats))
        return MOE_EINVAL;
    Workspace wl;
    if ((rc = check_ws(dm, workspace, workspace_bytes, &wl)) != MOE_OK)
        return rc;
    return hip_status(launch_dispatch(dm, x, topk_idx, topk_w, send_buf, send_scale, slot,
                                      expert_count, expert_kept,
                                      expert_offset, rank_rows, stats, (char *)workspace, wl,
                                      static_cast<hipStream_t>(stream)));
}

MOE_EXPORT int moe_dispatch_noalloc(const moe_shape *shape, const uint16_t *x,
                                    const int32_t *topk_idx, const float *topk_w, void *send_buf,
                                    float *send_scale, int32_t *slot, int32_t *expert_count,
                                    int32_t *expert_kept, int32_t *expert_offset,
                                    int32_t *rank_rows, moe_stats *stats, void *stream)
{
    Dims dm;
    const int rc = make_dims(shape, &dm);
    if (rc != MOE_OK)
        return rc;
    const bool need_w = dm.drop_policy == 1 && dm.capacity >= 0;
    if (need_w ? bad_ptr(topk_w, dm.T) : bad_opt_ptr(topk_w))
        return MOE_EINVAL;
    if (bad_scale(dm, send_scale))
        return MOE_EINVAL;
    if (bad_ptr(x, dm.T) || bad_ptr(topk_idx, dm.T) || bad_ptr(send_buf, dm.send_rows) ||
        bad_ptr(slot, dm.T) || bad_ptr(expert_count) || bad_ptr(expert_kept) ||
        bad_ptr(expert_offset) || bad_ptr(rank_rows) || bad_ptr(stats))
        return MOE_EINVAL;
    const Workspace wl = dispatch_layout(dm);
    if (wl.total > MOE_DISPATCH_SCRATCH_BYTES)
        return MOE_ESCRATCH;
    hipError_t e;
    char *ws = device_scratch(&e);
    if (!ws)
        return MOE_EHIP;
    return hip_status(launch_dispatch(dm, x, topk_idx, topk_w, send_buf, send_scale, slot,
                                      expert_count, expert_kept, expert_offset, rank_rows, stats,
                                      ws, wl, static_cast<hipStream_t>(stream)));
}

MOE_EXPORT int moe_expert_ffn(const moe_shape *shape, const void *send_buf,
                              const float *send_scale, const int32_t *expert_offset,
                              const int32_t *expert_kept,
                              const uint16_t *w1, const uint16_t *w3, const uint16_t *w2,
                              uint16_t *expert_out, void *workspace, size_t workspace_bytes,
                              void *stream)
{
    Dims dm;
    int rc = make_dims(shape, &dm);
    if (rc != MOE_OK)
        return rc;
    if (bad_ptr(send_buf, dm.send_rows) || bad_ptr(expert_offset) || bad_ptr(expert_kept) ||
        bad_ptr(w1) || bad_ptr(w3) || bad_ptr(w2) || bad_ptr(expert_out, dm.send_rows) ||
        bad_scale(dm, send_scale))
        return MOE_EINVAL;
    Workspace wl;
    if ((rc = check_ws(dm, workspace, workspace_bytes, &wl)) != MOE_OK)
        return rc;
    hipStream_t st = static_cast<hipStream_t>(stream);
    uint16_t *h = reinterpret_cast<uint16_t *>((char *)workspace + wl.h);
    uint16_t *a_wide = reinterpret_cast<uint16_t *>((char *)workspace + wl.a_wide);
    hipError_t e = launch_gate_up(dm, send_buf, send_scale, expert_offset, expert_kept, w1, w3,
                                  h, a_wide, st);
    if (e == hipSuccess)
        e = launch_down(dm, h, expert_offset, expert_kept, w2, expert_out, st);
    return hip_status(e);
}

MOE_EXPORT int moe_expert_gate_up(const moe_shape *shape, const void *send_buf,
                                  const float *send_scale, const int32_t *expert_offset,
                                  const int32_t *expert_kept, const uint16_t *w1,
                                  const uint16_t *w3, uint16_t *h, void *workspace,
                                  size_t workspace_bytes, void *stream)
{
    Dims dm;
    int rc = make_dims(shape, &dm);
    if (rc != MOE_OK)
        return rc;
    if (bad_ptr(send_buf, dm.send_rows) || bad_ptr(expert_offset) || bad_ptr(expert_kept) ||
        bad_ptr(w1) || bad_ptr(w3) || bad_ptr(h, dm.send_rows) || bad_scale(dm, send_scale))
        return MOE_EINVAL;
    uint16_t *a_wide = nullptr; // the workspace is optional here
    if (workspace) {
        Workspace wl;
        if ((rc = check_ws(dm, workspace, workspace_bytes, &wl)) != MOE_OK)
            return rc;
        a_wide = reinterpret_cast<uint16_t *>((char *)workspace + wl.a_wide);
    }
    return hip_status(launch_gate_up(dm, send_buf, send_scale, expert_offset, expert_kept, w1,
                                     w3, h, a_wide, static_cast<hipStream_t>(stream)));
}

MOE_EXPORT int moe_expert_down(const moe_shape *shape, const uint16_t *h,
                               const int32_t *expert_offset, const int32_t *expert_kept,
                               const uint16_t *w2, uint16_t *expert_out, void *stream)
{
    Dims dm;
    const int rc = make_dims(shape, &dm);
    if (rc != MOE_OK)
        return rc;
    if (bad_ptr(h, dm.send_rows) || bad_ptr(expert_offset) || bad_ptr(expert_kept) ||
        bad_ptr(w2) || bad_ptr(expert_out, dm.send_rows))
        return MOE_EINVAL;
    return hip_status(launch_down(dm, h, expert_offset, expert_kept, w2, expert_out,
                                  static_cast<hipStream_t>(stream)));
}

MOE_EXPORT int moe_combine(const moe_shape *shape, const uint16_t *expert_out,
                           const int32_t *slot, const float *topk_w, const uint16_t *shared_out,
                           uint16_t *y, void *stream)
{
    Dims dm;
    const int rc = make_dims(shape, &dm);
    if (rc != MOE_OK)
        return rc;
    if (bad_ptr(expert_out, dm.send_rows) || bad_ptr(slot, dm.T) || bad_ptr(topk_w, dm.T) ||
        bad_ptr(y, dm.T) || bad_opt_ptr(shared_out))
        return MOE_EINVAL;
    return hip_status(launch_combine(dm, expert_out, slot, topk_w, shared_out, y,
                                     static_cast<hipStream_t>(stream)));
}

MOE_EXPORT int moe_shared_expert(const moe_shape *shape, const uint16_t *x, const uint16_t *w1s,
                                 const uint16_t *w3s, const uint16_t *w2s, uint16_t *shared_out,
                                 void *workspace, size_t workspace_bytes, void *stream)
{
    Dims dm;
    int rc = make_dims(shape, &dm);
    if (rc != MOE_OK)
        return rc;
    if (dm.shared_H == 0)
        return MOE_EINVAL;
    if (bad_ptr(x, dm.T) || bad_ptr(w1s) || bad_ptr(w3s) || bad_ptr(w2s) ||
        bad_ptr(shared_out, dm.T))
        return MOE_EINVAL;
    Workspace wl;
    if ((rc = check_ws(dm, workspace, workspace_bytes, &wl)) != MOE_OK)
        return rc;
    return hip_status(launch_shared_expert(dm, x, w1s, w3s, w2s, shared_out, (char *)workspace,
                                           wl, static_cast<hipStream_t>(stream)));
}

MOE_EXPORT int moe_layer_fwd(const moe_shape *shape, const uint16_t *x, const uint16_t *w_gate,
                             const float *logit_bias, const uint16_t *w1, const uint16_t *w3,
                             const uint16_t *w2, const uint16_t *w1s, const uint16_t *w3s,
                             const uint16_t *w2s, uint16_t *y, float *logits_out,
                             int32_t *topk_idx, float *topk_w, void *send_buf,
                             float *send_scale, int32_t *slot, int32_t *expert_count, int32_t *expert_kept, int32_t *expert_offset,
                             int32_t *rank_rows, moe_stats *stats, uint16_t *expert_out,
                             uint16_t *shared_out, void *workspace, size_t workspace_bytes,
                             void *stream)
{
    Dims dm;
    int rc = make_dims(shape, &dm);
    if (rc != MOE_OK)
        return rc;
    if (bad_ptr(x, dm.T) || bad_ptr(w_gate) || bad_ptr(w1) || bad_ptr(w3) || bad_ptr(w2) ||
        bad_ptr(y, dm.T) || bad_ptr(topk_idx, dm.T) || bad_ptr(topk_w, dm.T) ||
        bad_ptr(send_buf, dm.send_rows) || bad_ptr(slot, dm.T) || bad_ptr(expert_count) ||
        bad_ptr(expert_kept) || bad_ptr(expert_offset) || bad_ptr(rank_rows) ||
        bad_ptr(stats) || bad_ptr(expert_out, dm.send_rows) || bad_opt_ptr(logit_bias) ||
        bad_opt_ptr(logits_out) || bad_scale(dm, send_scale))
        return MOE_EINVAL;
    if (dm.shared_H > 0 ? (bad_ptr(w1s) || bad_ptr(w3s) || bad_ptr(w2s) || bad_ptr(shared_out, dm.T))
                        : (bad_opt_ptr(w1s) || bad_opt_ptr(w3s) || bad_opt_ptr(w2s) ||
                           bad_opt_ptr(shared_out)))
        return MOE_EINVAL;
    Workspace wl;
    if ((rc = check_ws(dm, workspace, workspace_bytes, &wl)) != MOE_OK)
        return rc;
    hipStream_t st = static_cast<hipStream_t>(stream);
    char *ws = (char *)workspace;
    hipError_t e =
        launch_route(dm, x, w_gate, logit_bias, logits_out, topk_idx, topk_w, ws, wl, st);
    if (e == hipSuccess)
        e = launch_dispatch(dm, x, topk_idx, topk_w, send_buf, send_scale, slot, expert_count,
                            expert_kept, expert_offset, rank_rows, stats, ws, wl, st);
    if (e == hipSuccess)
        e = launch_gate_up(dm, send_buf, send_scale, expert_offset, expert_kept, w1, w3,
                           reinterpret_cast<uint16_t *>(ws + wl.h),
                           reinterpret_cast<uint16_t *>(ws + wl.a_wide), st);
    if (e == hipSuccess)
        e = launch_down(dm, reinterpret_cast<const uint16_t *>(ws + wl.h), expert_offset,
                        expert_kept, w2, expert_out, st);
    const bool shared = dm.shared_H > 0;
    if (e == hipSuccess && shared)
        e = launch_shared_expert(dm, x, w1s, w3s, w2s, shared_out, ws, wl, st);
    if (e == hipSuccess)
        e = launch_combine(dm, expert_out, slot, topk_w, shared ? shared_out : nullptr, y, st);
    return hip_status(e);
}

MOE_EXPORT int moe_fp8_rows_to_bf16(const void *codes, const float *scales, int64_t rows,
                                    int32_t d, uint16_t *out, void *stream)
{
    if (rows < 0 || d <= 0 || d % 16 != 0 || rows * (int64_t)(d / 4) > (int64_t)INT32_MAX * 256)
        return MOE_EINVAL;
    if (bad_ptr(codes, rows) || bad_ptr(scales, rows) || bad_ptr(out, rows))
        return MOE_EINVAL;
    return hip_status(launch_fp8_rows_to_bf16(static_cast<const uint8_t *>(codes), scales, rows,
                                              d, out, static_cast<hipStream_t>(stream)));
}

MOE_EXPORT int moe_stream_read(const void *src, size_t bytes, uint32_t *sink, void *stream)
{
    if (bytes % 16 != 0 || bad_ptr(src, (long long)(bytes / 16)) || bad_ptr(sink))
        return MOE_EINVAL;
    return hip_status(launch_stream_read(src, bytes, sink, static_cast<hipStream_t>(stream)));
}

MOE_EXPORT int moe_stream_write(void *dst, size_t bytes, uint32_t value, void *stream)
{
    if (bytes % 16 != 0 || bad_ptr(dst, (long long)(bytes / 16)))
        return MOE_EINVAL;
    return hip_status(launch_stream_write(dst, bytes, value, static_cast<hipStream_t>(stream)));
}

MOE_EXPORT int moe_stream_gather(const void *rows, int64_t nrows, int32_t d, const int32_t *slot,
                                 int64_t T, int32_t k, void *out, void *stream)
{
    if (nrows < 0 || d <= 0 || d % 8 != 0 || T < 0 || T > INT32_MAX || k < 1 ||
        (long long)T * k > INT32_MAX)
        return MOE_EINVAL;
    if (bad_ptr(rows, nrows) || bad_ptr(slot, T) || bad_ptr(out, T))
        return MOE_EINVAL;
    return hip_status(launch_stream_gather(rows, nrows, d, slot, (int)T, k, out,
                                           static_cast<hipStream_t>(stream)));
}

MOE_EXPORT const char *moe_status_str(int status)
{
    switch (status) {
    case MOE_OK:
        return "ok";
    case MOE_EINVAL:
        return "invalid argument";
    case MOE_EUNSUPPORTED:
        return "unsupported shape";
    case MOE_EWORKSPACE:
        return "workspace missing or too small";
    case MOE_EHIP:
        return "HIP launch error";
    case MOE_ESCRATCH:
        return "shape needs more dispatch scratch than the static array holds";
    default:
        return "unknown status";
    }
}
