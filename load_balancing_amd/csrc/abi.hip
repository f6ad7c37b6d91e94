// abi.hip -- the extern "C" entry points of libmoonep: argument validation on
// the host, then the launches.  Every call is asynchronous on the caller's
// stream except moonep_read_error.  The operations each call performs are
// described, with the pages that define them, in include/moonep.h.
#include <stdint.h>
#include <string.h>

#include <mutex>

#include "moonep_internal.hpp"

namespace moonep {
int launch_route_stats(const moonep_shape &s, const int32_t *topk, int32_t *counts, float *maxvio,
                       void *ws, hipStream_t st);
int launch_plan(const moonep_shape &s, const int32_t *topk, const int32_t *counts, void *ws,
                int32_t *plan, int32_t *slot_of, int32_t *src_of_slot, hipStream_t st,
                int32_t policy);
size_t plan_lds_bytes(int32_t E, int32_t R);
int launch_dispatch(const moonep_shape &s, const uint16_t *x, const int32_t *slot_of, uint16_t *buf,
                    hipStream_t st);
int launch_combine(const moonep_shape &s, const uint16_t *out, const float *gates,
                   const int32_t *slot_of, uint16_t *y, hipStream_t st);
int launch_dispatch_bwd(const moonep_shape &s, const uint16_t *d_buf, const int32_t *slot_of,
                        uint16_t *dx, hipStream_t st);
int launch_combine_bwd(const moonep_shape &s, const uint16_t *dy, const uint16_t *out,
                       const float *gates, const int32_t *slot_of, uint16_t *d_out, float *d_gates,
                       hipStream_t st);
int launch_replica_reduce(const moonep_shape &s, const int32_t *plan, int64_t G, float *home,
                          float *rep, int grid, hipStream_t st);
int launch_weight_slots(const moonep_shape &s, const int32_t *plan, int32_t B, int32_t *wslot,
                        hipStream_t st);
int launch_prefetch(const moonep_shape &s, const int32_t *plan, const int32_t *wslot, int32_t B,
                    int64_t wbytes, const void *w_home, void *pool, int grid, hipStream_t st);
int gemm_out_align();
int launch_expert_gemm(const moonep_shape &s, const int32_t *plan, const int32_t *wslot, int32_t B,
                       int32_t in_dim, int32_t out_dim, const uint16_t *x, const uint16_t *w_home,
                       const uint16_t *pool, int64_t w_stride, int64_t w_offset, uint16_t *y,
                       hipStream_t st);
}  // namespace moonep

using namespace moonep;

// Scratch of moonep_plan_noalloc: the route_stats -> plan workspace of any
// valid shape (the 256-byte control block plus E x nseg int32 counts, with
// E <= 1024 and at most 2048 wave segments), one copy per device, held until
// the process ends.  In host code this name is not a device address: the
// address comes from hipGetSymbolAddress, once per device (static_scratch).
constexpr size_t kStaticScratchBytes = kCtlBytes + (size_t)4 * kMaxExperts * kMaxSegments;
static_assert(kStaticScratchBytes == (size_t)MOONEP_NOALLOC_SCRATCH_BYTES, "scratch size");
static __device__ __align__(256) uint8_t scratch[kStaticScratchBytes];

namespace {

constexpr int kMaxDevices = 64;
std::mutex scratch_mu;
void *scratch_ptr[kMaxDevices] = {};

// Device address of the current device's copy of `scratch`.
int static_scratch(void **out)
{
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices)
        return MOONEP_ERR_HIP;
    std::lock_guard<std::mutex> lock(scratch_mu);
    if (!scratch_ptr[dev]) {
        void *p = nullptr;
        if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess || !p)
            return MOONEP_ERR_HIP;
        scratch_ptr[dev] = p;
    }
    *out = scratch_ptr[dev];
    return MOONEP_OK;
}

bool aligned(const void *p, size_t a) { return ((uintptr_t)p % a) == 0; }

// [a, a + na) and [b, b + nb) share a byte.
bool overlap(const void *a, size_t na, const void *b, size_t nb)
{
    const uintptr_t x = (uintptr_t)a, y = (uintptr_t)b;
    return na && nb && x < y + nb && y < x + na;
}

int shape_status(const moonep_shape *s)
{
    if (!s)
        return MOONEP_ERR_NULL_PTR;
    if (s->R < 1 || s->E < 1 || s->S < 0 || s->K < 1 || s->H < 8)
        return MOONEP_ERR_INVALID_SHAPE;
    if (s->E % s->R != 0 || s->K > s->E || s->H % 8 != 0)
        return MOONEP_ERR_INVALID_SHAPE;
    if (s->E > kMaxExperts || s->R > kMaxRanks)
        return MOONEP_ERR_INVALID_SHAPE;
    if ((int64_t)s->R * s->S * s->K >= ((int64_t)1 << 31))
        return MOONEP_ERR_INVALID_SHAPE;
    return MOONEP_OK;
}

int64_t n_entries(const moonep_shape *s) { return (int64_t)s->R * s->S * s->K; }
int64_t n_tokens(const moonep_shape *s) { return (int64_t)s->R * s->S; }

// Pointers may be NULL only when the array they name is empty.
bool present(const void *p, int64_t n) { return p != nullptr || n == 0; }

}  // namespace

extern "C" {

int moonep_check_shape(const moonep_shape *shape) { return shape_status(shape); }

size_t moonep_workspace_bytes(const moonep_shape *shape)
{
    if (shape_status(shape) != MOONEP_OK)
        return 0;
    return ws_layout(*shape).bytes;
}

int moonep_plan_layout_of(const moonep_shape *shape, moonep_plan_layout *layout)
{
    const int rc = shape_status(shape);
    if (rc != MOONEP_OK)
        return rc;
    if (!layout)
        return MOONEP_ERR_NULL_PTR;
    const PlanLayout p = plan_layout(shape->E, shape->R);
    layout->words = p.words;
    layout->cap = p.cap;
    layout->header = p.header;
    layout->rep_expert = p.rep_expert;
    layout->rep_host = p.rep_host;
    layout->rep_count = p.rep_count;
    layout->rep_spill_off = p.rep_spill_off;
    layout->rep_row_off = p.rep_row_off;
    layout->spill = p.spill;
    layout->keep = p.keep;
    layout->home_row_off = p.home_row_off;
    layout->rep_first = p.rep_first;
    layout->rep_cnt = p.rep_cnt;
    layout->exp_rep_list = p.exp_rep_list;
    layout->load = p.load;
    layout->rank_rep_first = p.rank_rep_first;
    layout->rank_rep_cnt = p.rank_rep_cnt;
    return MOONEP_OK;
}

size_t moonep_plan_bytes(const moonep_shape *shape)
{
    if (shape_status(shape) != MOONEP_OK)
        return 0;
    return (size_t)plan_layout(shape->E, shape->R).words * 4;
}

int moonep_route_stats(const moonep_shape *shape, const int32_t *topk_idx, int32_t *expert_counts,
                       float *maxvio, void *workspace, size_t workspace_bytes, void *stream)
{
    int rc = shape_status(shape);
    if (rc != MOONEP_OK)
        return rc;
    const int64_t nk = n_entries(shape);
    if (!present(topk_idx, nk) || !expert_counts || !maxvio || !workspace)
        return MOONEP_ERR_NULL_PTR;
    if (!aligned(topk_idx, 4) || !aligned(expert_counts, 4) || !aligned(maxvio, 4) ||
        !aligned(workspace, 16))
        return MOONEP_ERR_MISALIGNED;
    if (workspace_bytes < ws_layout(*shape).bytes)
        return MOONEP_ERR_WORKSPACE;
    return launch_route_stats(*shape, topk_idx, expert_counts, maxvio, workspace,
                              (hipStream_t)stream);
}

namespace {

int plan_with_policy(const moonep_shape *shape, const int32_t *topk_idx,
                     const int32_t *expert_counts, void *workspace, size_t workspace_bytes,
                     int32_t *plan, int32_t *slot_of, int32_t *src_of_slot, void *stream,
                     int32_t policy)
{
    int rc = shape_status(shape);
    if (rc != MOONEP_OK)
        return rc;
    const int64_t nk = n_entries(shape);
    if (!present(topk_idx, nk) || !expert_counts || !workspace || !plan ||
        !present(slot_of, nk) || !present(src_of_slot, nk))
        return MOONEP_ERR_NULL_PTR;
    if (!aligned(topk_idx, 4) || !aligned(expert_counts, 4) || !aligned(plan, 4) ||
        !aligned(slot_of, 4) || !aligned(src_of_slot, 4) || !aligned(workspace, 16))
        return MOONEP_ERR_MISALIGNED;
    if (workspace_bytes < ws_layout(*shape).bytes)
        return MOONEP_ERR_WORKSPACE;
    if (overlap(slot_of, nk * 4, src_of_slot, nk * 4))
        return MOONEP_ERR_ALIAS;
    return launch_plan(*shape, topk_idx, expert_counts, workspace, plan, slot_of, src_of_slot,
                       (hipStream_t)stream, policy);
}

}  // namespace

int moonep_plan(const moonep_shape *shape, const int32_t *topk_idx, const int32_t *expert_counts,
                void *workspace, size_t workspace_bytes, int32_t *plan, int32_t *slot_of,
                int32_t *src_of_slot, void *stream)
{
    return plan_with_policy(shape, topk_idx, expert_counts, workspace, workspace_bytes, plan,
                            slot_of, src_of_slot, stream, 0);
}

int moonep_plan_largest_first(const moonep_shape *shape, const int32_t *topk_idx,
                              const int32_t *expert_counts, void *workspace,
                              size_t workspace_bytes, int32_t *plan, int32_t *slot_of,
                              int32_t *src_of_slot, void *stream)
{
    return plan_with_policy(shape, topk_idx, expert_counts, workspace, workspace_bytes, plan,
                            slot_of, src_of_slot, stream, 1);
}

int moonep_plan_noalloc(const moonep_shape *shape, const int32_t *topk_idx, int32_t *expert_counts,
                        float *maxvio, int32_t *plan, int32_t *slot_of, int32_t *src_of_slot,
                        void *stream)
{
    int rc = shape_status(shape);
    if (rc != MOONEP_OK)
        return rc;
    const int64_t nk = n_entries(shape);
    if (!present(topk_idx, nk) || !expert_counts || !maxvio || !plan || !present(slot_of, nk) ||
        !present(src_of_slot, nk))
        return MOONEP_ERR_NULL_PTR;
    if (!aligned(topk_idx, 4) || !aligned(expert_counts, 4) || !aligned(maxvio, 4) ||
        !aligned(plan, 4) || !aligned(slot_of, 4) || !aligned(src_of_slot, 4))
        return MOONEP_ERR_MISALIGNED;
    if (overlap(slot_of, nk * 4, src_of_slot, nk * 4))
        return MOONEP_ERR_ALIAS;
    if (ws_layout(*shape).bytes > kStaticScratchBytes)
        return MOONEP_ERR_WORKSPACE;
    void *ws = nullptr;
    if ((rc = static_scratch(&ws)) != MOONEP_OK)
        return rc;
    const hipStream_t st = (hipStream_t)stream;
    if ((rc = launch_route_stats(*shape, topk_idx, expert_counts, maxvio, ws, st)) != MOONEP_OK)
        return rc;
    return launch_plan(*shape, topk_idx, expert_counts, ws, plan, slot_of, src_of_slot, st, 0);
}

int moonep_dispatch(const moonep_shape *shape, const uint16_t *x, const int32_t *slot_of,
                    uint16_t *buf, void *stream)
{
    int rc = shape_status(shape);
    if (rc != MOONEP_OK)
        return rc;
    const int64_t nk = n_entries(shape), nt = n_tokens(shape);
    if (!present(x, nt) || !present(slot_of, nk) || !present(buf, nk))
        return MOONEP_ERR_NULL_PTR;
    if (!aligned(x, 16) || !aligned(buf, 16) || !aligned(slot_of, 4))
        return MOONEP_ERR_MISALIGNED;
    const size_t row = (size_t)shape->H * 2;
    if (overlap(x, nt * row, buf, nk * row))
        return MOONEP_ERR_ALIAS;
    return launch_dispatch(*shape, x, slot_of, buf, (hipStream_t)stream);
}

int moonep_combine(const moonep_shape *shape, const uint16_t *expert_out, const float *gates,
                   const int32_t *slot_of, uint16_t *y, void *stream)
{
    int rc = shape_status(shape);
    if (rc != MOONEP_OK)
        return rc;
    const int64_t nk = n_entries(shape), nt = n_tokens(shape);
    if (!present(expert_out, nk) || !present(gates, nk) || !present(slot_of, nk) ||
        !present(y, nt))
        return MOONEP_ERR_NULL_PTR;
    if (!aligned(expert_out, 16) || !aligned(y, 16) || !aligned(gates, 4) || !aligned(slot_of, 4))
        return MOONEP_ERR_MISALIGNED;
    const size_t row = (size_t)shape->H * 2;
    if (overlap(expert_out, nk * row, y, nt * row))
        return MOONEP_ERR_ALIAS;
    return launch_combine(*shape, expert_out, gates, slot_of, y, (hipStream_t)stream);
}

int moonep_combine_bwd(const moonep_shape *shape, const uint16_t *dy, const uint16_t *expert_out,
                       const float *gates, const int32_t *slot_of, uint16_t *d_out,
                       float *d_gates, void *stream)
{
    int rc = shape_status(shape);
    if (rc != MOONEP_OK)
        return rc;
    const int64_t nk = n_entries(shape), nt = n_tokens(shape);
    if (!present(dy, nt) || !present(expert_out, nk) || !present(gates, nk) ||
        !present(slot_of, nk) || !present(d_out, nk) || !present(d_gates, nk))
        return MOONEP_ERR_NULL_PTR;
    if (!aligned(dy, 16) || !aligned(expert_out, 16) || !aligned(d_out, 16) || !aligned(gates, 4) ||
        !aligned(slot_of, 4) || !aligned(d_gates, 4))
        return MOONEP_ERR_MISALIGNED;
    const size_t row = (size_t)shape->H * 2;
    if (overlap(d_out, nk * row, dy, nt * row) || overlap(d_out, nk * row, expert_out, nk * row))
        return MOONEP_ERR_ALIAS;
    return launch_combine_bwd(*shape, dy, expert_out, gates, slot_of, d_out, d_gates,
                              (hipStream_t)stream);
}

int moonep_dispatch_bwd(const moonep_shape *shape, const uint16_t *d_buf, const int32_t *slot_of,
                        uint16_t *dx, void *stream)
{
    int rc = shape_status(shape);
    if (rc != MOONEP_OK)
        return rc;
    const int64_t nk = n_entries(shape), nt = n_tokens(shape);
    if (!present(d_buf, nk) || !present(slot_of, nk) || !present(dx, nt))
        return MOONEP_ERR_NULL_PTR;
    if (!aligned(d_buf, 16) || !aligned(dx, 16) || !aligned(slot_of, 4))
        return MOONEP_ERR_MISALIGNED;
    const size_t row = (size_t)shape->H * 2;
    if (overlap(d_buf, nk * row, dx, nt * row))
        return MOONEP_ERR_ALIAS;
    return launch_dispatch_bwd(*shape, d_buf, slot_of, dx, (hipStream_t)stream);
}

int moonep_replica_grad_reduce(const moonep_shape *shape, const int32_t *plan, int64_t G,
                               float *home_grads, float *replica_grads, void *stream)
{
    int rc = shape_status(shape);
    if (rc != MOONEP_OK)
        return rc;
    if (G < 0)
        return MOONEP_ERR_ARG;
    if (!plan || !present(home_grads, G) || !present(replica_grads, G))
        return MOONEP_ERR_NULL_PTR;
    if (!aligned(plan, 4) || !aligned(home_grads, 4) || !aligned(replica_grads, 4))
        return MOONEP_ERR_MISALIGNED;
    const size_t hb = (size_t)shape->E * (size_t)G * 4;
    const size_t rb = (size_t)(shape->E + shape->R) * (size_t)G * 4;
    if (overlap(home_grads, hb, replica_grads, rb))
        return MOONEP_ERR_ALIAS;
    int dev = 0, cus = 0;
    if (hipGetDevice(&dev) != hipSuccess ||
        hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess)
        return MOONEP_ERR_HIP;
    return launch_replica_reduce(*shape, plan, G, home_grads, replica_grads, cus * 4,
                                 (hipStream_t)stream);
}

int moonep_weight_slots(const moonep_shape *shape, const int32_t *plan, int32_t B, int32_t *wslot,
                        void *stream)
{
    int rc = shape_status(shape);
    if (rc != MOONEP_OK)
        return rc;
    if (B < 0 || (int64_t)shape->R * B >= ((int64_t)1 << 31))
        return MOONEP_ERR_ARG;
    if (!plan || !wslot)
        return MOONEP_ERR_NULL_PTR;
    if (!aligned(plan, 4) || !aligned(wslot, 4))
        return MOONEP_ERR_MISALIGNED;
    return launch_weight_slots(*shape, plan, B, wslot, (hipStream_t)stream);
}

int moonep_prefetch_weights(const moonep_shape *shape, const int32_t *plan, const int32_t *wslot,
                            int32_t B, int64_t wbytes, const void *w_home, void *pool, void *stream)
{
    int rc = shape_status(shape);
    if (rc != MOONEP_OK)
        return rc;
    if (B < 0 || (int64_t)shape->R * B >= ((int64_t)1 << 31) || wbytes < 0 || wbytes % 16 != 0)
        return MOONEP_ERR_ARG;
    const int64_t pool_rows = (int64_t)shape->R * B;
    if (!plan || !wslot || !present(w_home, wbytes) || !present(pool, pool_rows * wbytes))
        return MOONEP_ERR_NULL_PTR;
    if (!aligned(plan, 4) || !aligned(wslot, 4) || !aligned(w_home, 16) || !aligned(pool, 16))
        return MOONEP_ERR_MISALIGNED;
    if (overlap(w_home, (size_t)shape->E * (size_t)wbytes, pool, (size_t)pool_rows * (size_t)wbytes))
        return MOONEP_ERR_ALIAS;
    int dev = 0, cus = 0;
    if (hipGetDevice(&dev) != hipSuccess ||
        hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess)
        return MOONEP_ERR_HIP;
    return launch_prefetch(*shape, plan, wslot, B, wbytes, w_home, pool, cus * 4,
                           (hipStream_t)stream);
}

int moonep_expert_gemm(const moonep_shape *shape, const int32_t *plan, const int32_t *wslot,
                       int32_t B, int32_t in_dim, int32_t out_dim, const uint16_t *x,
                       const uint16_t *w_home, const uint16_t *pool, int64_t w_stride,
                       int64_t w_offset, uint16_t *y, void *stream)
{
    int rc = shape_status(shape);
    if (rc != MOONEP_OK)
        return rc;
    // the kernel addresses a row of a tile by a 32-bit byte offset: 256 rows of in_dim bf16
    constexpr int32_t kMaxInDim = 1 << 22;
    if (B < 0 || (int64_t)shape->R * B >= ((int64_t)1 << 31) || in_dim <= 0 || in_dim % 64 != 0 ||
        in_dim > kMaxInDim || out_dim <= 0 || out_dim % gemm_out_align() != 0 ||
        w_stride % 8 != 0 || w_offset < 0 || w_offset % 8 != 0 ||
        w_offset + (int64_t)out_dim * in_dim > w_stride)
        return MOONEP_ERR_ARG;
    const int64_t rows = n_entries(shape);
    const int64_t pool_rows = (int64_t)shape->R * B;
    if (!plan || !wslot || !w_home || !present(x, rows) || !present(y, rows) ||
        !present(pool, pool_rows))
        return MOONEP_ERR_NULL_PTR;
    if (!aligned(plan, 4) || !aligned(wslot, 4) || !aligned(x, 16) || !aligned(y, 16) ||
        !aligned(w_home, 16) || !aligned(pool, 16))
        return MOONEP_ERR_MISALIGNED;
    const size_t yb = (size_t)rows * out_dim * 2;
    if (overlap(y, yb, x, (size_t)rows * in_dim * 2) ||
        overlap(y, yb, w_home, (size_t)shape->E * (size_t)w_stride * 2) ||
        overlap(y, yb, pool, (size_t)pool_rows * (size_t)w_stride * 2))
        return MOONEP_ERR_ALIAS;
    return launch_expert_gemm(*shape, plan, wslot, B, in_dim, out_dim, x, w_home, pool, w_stride,
                              w_offset, y, (hipStream_t)stream);
}

int moonep_read_error(void *workspace, size_t workspace_bytes, int32_t *host_code, void *stream)
{
    if (!workspace || !host_code)
        return MOONEP_ERR_NULL_PTR;
    if (workspace_bytes < kCtlBytes)
        return MOONEP_ERR_WORKSPACE;
    hipStream_t st = (hipStream_t)stream;
    int32_t v = 0;
    if (hipMemcpyAsync(&v, (int32_t *)workspace + kCtlError, 4, hipMemcpyDeviceToHost, st) !=
            hipSuccess ||
        hipStreamSynchronize(st) != hipSuccess)
        return MOONEP_ERR_HIP;
    *host_code = v;
    if (v != 0) {
        if (hipMemsetAsync((int32_t *)workspace + kCtlError, 0, 4, st) != hipSuccess ||
            hipStreamSynchronize(st) != hipSuccess)
            return MOONEP_ERR_HIP;
    }
    return MOONEP_OK;
}

}  // extern "C"
