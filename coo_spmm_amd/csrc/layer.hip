// layer.hip -- the C ABI of snack.h: layer lifetime, queries and the
// forward / backward / drop-regrow entry points.  Host code only: it checks
// arguments, owns the device buffers and launches the kernels of the other
// translation units on the caller's stream.
#include "internal.h"

#include <limits.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

using namespace snack;

namespace snack {

void report_hip_error(hipError_t e, const char* expr, const char* file, int line)
{
    static const bool on = getenv("SNACK_DEBUG") != nullptr;
    if (on) fprintf(stderr, "snack: %s failed at %s:%d: %s\n", expr, file, line, hipGetErrorString(e));
}

snack_status layer_alloc(snack_layer* L, void** p, size_t bytes)
{
    *p = nullptr;
    if (bytes == 0) bytes = 256;
    bytes = (bytes + 255) & ~(size_t)255;
    if (hipMalloc(p, bytes) != hipSuccess) {
        *p = nullptr;
        (void)hipGetLastError();
        return SNACK_ERR_ALLOC;
    }
    L->allocations.push_back(*p);
    L->device_bytes += bytes;
    return SNACK_OK;
}

}  // namespace snack

namespace {

void free_layer(snack_layer* L)
{
    if (!L) return;
    (void)hipDeviceSynchronize();
    for (void* p : L->allocations) (void)hipFree(p);
    if (L->ws) (void)hipFree(L->ws);
    if (L->host_res) (void)hipHostFree(L->host_res);
    if (L->grow_ev) (void)hipEventDestroy(L->grow_ev);
    delete L;
}

inline hipStream_t as_stream(snack_stream s) { return reinterpret_cast<hipStream_t>(s); }

size_t ws_need(const snack_layer* L, const BatchPlan& p)
{
    const size_t a = (((size_t)L->K * p.bp * 4) + 255) & ~(size_t)255;
    const size_t b = (((size_t)L->M * p.bp * 4) + 255) & ~(size_t)255;
    return a + b + tile_part_bytes(L, p) + wide_dw_bytes(L, p);
}

// grow the workspace to hold plan p (never shrinks); the new buffer is
// allocated before the old one is released, so a failed grow keeps the old
// reserve
snack_status ensure_ws(snack_layer* L, const BatchPlan& p)
{
    const size_t need = ws_need(L, p);
    if (need <= L->ws_bytes) return SNACK_OK;
    void* p2 = nullptr;
    if (hipMalloc(&p2, need) != hipSuccess) {
        (void)hipGetLastError();
        return SNACK_ERR_ALLOC;
    }
    if (L->ws) {
        // work queued on any stream may still read the old buffer
        const hipError_t e = hipDeviceSynchronize();
        if (e != hipSuccess) {
            report_hip_error(e, "hipDeviceSynchronize", __FILE__, __LINE__);
            (void)hipFree(p2);
            return SNACK_ERR_HIP;
        }
        (void)hipFree(L->ws);
        L->device_bytes -= L->ws_bytes;
    }
    L->ws = (float*)p2;
    L->ws_bytes = need;
    L->device_bytes += need;
    return SNACK_OK;
}

// the compute entry points never allocate: a batch plan whose workspace is not
// reserved is refused before anything is launched
snack_status ws_check(const snack_layer* L, const BatchPlan& p)
{
    return ws_need(L, p) <= L->ws_bytes ? SNACK_OK : SNACK_ERR_WORKSPACE;
}

// the largest workspace of any batch plan up to max_batch (the slice-tiled
// passes' buffers are only taken below size limits, so a smaller batch can
// need more than max_batch itself): one batch per plan, at most
// kMaxBatch / 64 + 7 of them
snack_status reserve_ws(snack_layer* L, int32_t max_batch)
{
    BatchPlan best = plan_batch(1);
    size_t need = 0;
    for (int32_t b = 1;;) {
        const BatchPlan p = plan_batch(b);
        const size_t n = ws_need(L, p);
        if (n > need) {
            need = n;
            best = p;
        }
        if (b >= max_batch) break;
        const int32_t next = b < 64 ? 2 * b : b + 64;
        b = next < max_batch ? next : max_batch;
    }
    return ensure_ws(L, best);
}

float* ws_x(snack_layer* L) { return L->ws; }

}  // namespace

// partial sums of the slice-tiled kernels: after both feature-major copies
float* snack::ws_part(const snack_layer* L, const BatchPlan& p)
{
    const size_t a = (((size_t)L->K * p.bp * 4) + 255) & ~(size_t)255;
    const size_t b = (((size_t)L->M * p.bp * 4) + 255) & ~(size_t)255;
    return (float*)((char*)L->ws + a + b);
}

namespace {

// the per-tile dW slabs of the several-tile column pass: after the partial sums
float* ws_dw_slabs(snack_layer* L, const BatchPlan& p)
{
    return (float*)((char*)ws_part(L, p) + tile_part_bytes(L, p));
}

float* ws_dy(snack_layer* L, const BatchPlan& p)
{
    const size_t a = (((size_t)L->K * p.bp * 4) + 255) & ~(size_t)255;
    return (float*)((char*)L->ws + a);
}

}  // namespace

extern "C" const char* snack_status_string(snack_status s)
{
    switch (s) {
    case SNACK_OK: return "ok";
    case SNACK_ERR_INVALID_ARG: return "invalid argument";
    case SNACK_ERR_INDEX_RANGE: return "index out of range";
    case SNACK_ERR_DUPLICATE: return "duplicate position";
    case SNACK_ERR_ALLOC: return "device allocation failed";
    case SNACK_ERR_HIP: return "HIP runtime error";
    case SNACK_ERR_UNSUPPORTED: return "unsupported size";
    case SNACK_ERR_WORKSPACE: return "batch exceeds the reserved workspace (snack_layer_reserve)";
    }
    return "unknown status";
}

extern "C" snack_status snack_layer_create(int32_t M, int32_t K, int64_t nnz, const int32_t* rows,
                                           const int32_t* cols, const float* vals, uint64_t seed,
                                           snack_stream stream, snack_layer** out)
{
    if (!out) return SNACK_ERR_INVALID_ARG;
    *out = nullptr;
    if (M < 1 || K < 1 || nnz < 0) return SNACK_ERR_INVALID_ARG;
    if ((uint64_t)nnz > (uint64_t)M * (uint64_t)K) return SNACK_ERR_INVALID_ARG;
    if (nnz > (int64_t)INT_MAX - 4 * kPad) return SNACK_ERR_UNSUPPORTED;
    if (M > INT_MAX - 2 || K > INT_MAX - 2) return SNACK_ERR_UNSUPPORTED;
    if (nnz > 0 && (!rows || !cols)) return SNACK_ERR_INVALID_ARG;
    hipStream_t s = as_stream(stream);

    snack_layer* L = new snack_layer();
    {
        const hipError_t e = hipGetDevice(&L->device);
        if (e != hipSuccess) {
            report_hip_error(e, "hipGetDevice", __FILE__, __LINE__);
            delete L;
            return SNACK_ERR_HIP;
        }
    }
    {
        int lds = 0, cus = 0;
        const hipError_t e1 = hipDeviceGetAttribute(&lds, hipDeviceAttributeMaxSharedMemoryPerBlock, L->device);
        const hipError_t e2 = hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, L->device);
        if (e1 != hipSuccess || e2 != hipSuccess) {
            report_hip_error(e1 != hipSuccess ? e1 : e2, "hipDeviceGetAttribute", __FILE__, __LINE__);
            delete L;
            return SNACK_ERR_HIP;
        }
        L->lds_bytes = lds;
        L->cus = cus;
    }
    L->M = M;
    L->K = K;
    L->nnz = nnz;
    L->seed = seed;
    if (const char* e = getenv("SNACK_GROW_BUCKET_CAP")) {
        const long c = strtol(e, nullptr, 10);
        if (c > 0 && c < INT_MAX) L->grow_cap_max = (int32_t)c;
    }
    L->epoch = 0;
    L->cap = ((nnz + 255) / 256) * 256 + kPad;

    auto fail = [&](snack_status st) {
        free_layer(L);
        return st;
    };
    const size_t nb4 = (size_t)L->cap * 4;
    void* p = nullptr;
#define ALLOC(field, type, bytes)                                     \
    do {                                                              \
        snack_status _s = layer_alloc(L, &p, (bytes));                \
        if (_s != SNACK_OK) return fail(_s);                          \
        L->field = (type)p;                                           \
        hipError_t _e = hipMemsetAsync(p, 0, (bytes), s);             \
        if (_e != hipSuccess) {                                       \
            report_hip_error(_e, "hipMemsetAsync", __FILE__, __LINE__); \
            return fail(SNACK_ERR_HIP);                               \
        }                                                             \
    } while (0)
    ALLOC(rows, int32_t*, nb4);
    ALLOC(cols, int32_t*, nb4);
    ALLOC(vals, float*, nb4);
    ALLOC(iperm, int32_t*, nb4);
    ALLOC(rows_t, int32_t*, nb4);
    ALLOC(vals_t, float*, nb4);
    ALLOC(dwt, float*, nb4);
    ALLOC(row_ptr, int32_t*, ((size_t)M + 1) * 4);
    ALLOC(col_ptr, int32_t*, ((size_t)K + 1) * 4);
    ALLOC(flag, int32_t*, 64);

    {
        // chunks of up to kChunkWork units, smaller for small layers so that the
        // chunk-per-wavefront kernels still have about kChunkTarget chunks
        const int64_t w = (nnz + (M > K ? M : K)) / kChunkTarget;
        L->chunk_work = (int32_t)(w > kChunkWork ? kChunkWork : (w < kChunkWorkMin ? kChunkWorkMin : w));
    }
    const int64_t nchf = (nnz + M + L->chunk_work - 1) / L->chunk_work;
    const int64_t ncht = (nnz + K + L->chunk_work - 1) / L->chunk_work;
    if (nchf > INT_MAX / 2 || ncht > INT_MAX / 2) return fail(SNACK_ERR_UNSUPPORTED);
    L->fwd.nkeys = M;
    L->fwd.nidx = K;
    L->fwd.idx = L->cols;
    L->fwd.vals = L->vals;
    L->fwd.ptr = L->row_ptr;
    L->fwd.nchunks = (int32_t)(nchf < 1 ? 1 : nchf);
    ALLOC(fwd.desc, int2*, ((size_t)L->fwd.nchunks + 1) * 8);
    ALLOC(fwd.empty_keys, int32_t*, (size_t)M * 4);
    ALLOC(fwd.n_empty, int32_t*, 4);
    L->tr.nkeys = K;
    L->tr.nidx = M;
    L->tr.idx = L->rows_t;
    L->tr.vals = L->vals_t;
    L->tr.ptr = L->col_ptr;
    L->tr.nchunks = (int32_t)(ncht < 1 ? 1 : ncht);
    // 16-bit copies of the gathered indices for the narrow-batch streams (cap is a multiple of 4)
    if (K <= kIdx16Max) ALLOC(fwd.idx16, uint16_t*, (size_t)L->cap * 2);
    if (K <= kIdx16Max) ALLOC(vals16, uint16_t*, (size_t)L->cap * 2);   // the inference forward's values
    if (M <= kIdx16Max) ALLOC(tr.idx16, uint16_t*, (size_t)L->cap * 2);
    ALLOC(tr.desc, int2*, ((size_t)L->tr.nchunks + 1) * 8);
    ALLOC(tr.empty_keys, int32_t*, (size_t)K * 4);
    ALLOC(tr.n_empty, int32_t*, 4);

    {
        snack_status _s = alloc_split_tables(L);
        if (_s != SNACK_OK) return fail(_s);
    }

    size_t scr = canon_scratch_bytes(L, nnz);
    const size_t pscr = prune_scratch_bytes(L);
    if (pscr > scr) scr = pscr;
    {
        snack_status _s = layer_alloc(L, &L->scratch, scr);
        if (_s != SNACK_OK) return fail(_s);
        L->scratch_bytes = scr;
    }
    // coherent pinned words the drop/regrow's kernels write its result into (system-scope stores)
    if (hipHostMalloc((void**)&L->host_res, 64, hipHostMallocMapped | hipHostMallocCoherent) != hipSuccess) {
        L->host_res = nullptr;
        return fail(SNACK_ERR_ALLOC);
    }
    if (hipHostGetDevicePointer((void**)&L->host_res_dev, L->host_res, 0) != hipSuccess) return fail(SNACK_ERR_HIP);
    if (hipEventCreateWithFlags(&L->grow_ev, hipEventDisableTiming) != hipSuccess) {
        L->grow_ev = nullptr;
        return fail(SNACK_ERR_HIP);
    }
#undef ALLOC

    snack_status st = canon_sort_input(L, rows, cols, vals, s);
    if (st != SNACK_OK) return fail(st);
    int32_t flag = 0;
    {
        hipError_t e = hipMemcpyAsync(&flag, L->flag, 4, hipMemcpyDeviceToHost, s);
        if (e == hipSuccess) e = hipStreamSynchronize(s);
        if (e != hipSuccess) {
            report_hip_error(e, "validation flag read", __FILE__, __LINE__);
            return fail(SNACK_ERR_HIP);
        }
    }
    if (flag & 1) return fail(SNACK_ERR_INDEX_RANGE);
    if (flag & 2) return fail(SNACK_ERR_DUPLICATE);
    st = canon_build_index(L, s);
    if (st != SNACK_OK) return fail(st);
    st = reserve_ws(L, kDefaultReserve);
    if (st != SNACK_OK) return fail(st);
    *out = L;
    return SNACK_OK;
}

extern "C" snack_status snack_layer_destroy(snack_layer* layer)
{
    free_layer(layer);
    return SNACK_OK;
}

extern "C" snack_status snack_layer_reserve(snack_layer* L, int32_t max_batch)
{
    if (!L || max_batch < 1) return SNACK_ERR_INVALID_ARG;
    if (max_batch > kMaxBatch) return SNACK_ERR_UNSUPPORTED;
    return reserve_ws(L, max_batch);
}

extern "C" snack_status snack_forward(snack_layer* L, const float* X, float* Y, int32_t B, snack_stream stream)
{
    if (!L || !X || !Y || B < 1) return SNACK_ERR_INVALID_ARG;
    if (B > kMaxBatch) return SNACK_ERR_UNSUPPORTED;
    hipStream_t s = as_stream(stream);
    const BatchPlan p = plan_batch(B);
    if (spmm_batch_major(L, p, true, false, false)) return spmm_forward(L, X, p, B, Y, s, true);
    const float* feat = X;
    if (p.bp > 1) {
        SNACK_CHECK(ws_check(L, p));
        SNACK_CHECK(transpose_pad(X, ws_x(L), L->K, nullptr, nullptr, 0, B, p.bp, s));
        feat = ws_x(L);
    }
    return spmm_forward(L, feat, p, B, Y, s);
}

namespace {

// the backward of snack_backward; with `step`, the column pass may also take the
// SGD step of vals_t in place (step->done tells whether it did).  x_ready /
// dy_ready: the workspace already holds the feature-major copy of X / dY for
// this batch plan (written by the forward of the same training step).
snack_status backward_impl(snack_layer* L, const float* X, const float* dY, float* dX, float* dW, int32_t B,
                           hipStream_t s, SgdStep* step, bool x_ready = false, bool dy_ready = false)
{
    const BatchPlan p = plan_batch(B);
    const bool rm = spmm_batch_major(L, p, false, dX != nullptr, dW != nullptr);
    const float* dyt = dY;
    const float* xt = X;
    if (p.bp > 1 && !rm) {
        SNACK_CHECK(ws_check(L, p));
        const float* xs = (dW && !x_ready) ? X : nullptr;
        if (!dy_ready) SNACK_CHECK(transpose_pad(dY, ws_dy(L, p), L->M, xs, ws_x(L), L->K, B, p.bp, s));
        else if (xs) SNACK_CHECK(transpose_pad(xs, ws_x(L), L->K, nullptr, nullptr, 0, B, p.bp, s));
        dyt = ws_dy(L, p);
        xt = ws_x(L);
    }
    if (dX && L->vals_t_stale) SNACK_CHECK(refresh_vals_t(L, s));
    L->dwt_valid = false;
    if (p.ntiles == 1) {
        // one launch: dX (+ dW in transposed order) over the column view, dW over the row view
        float* dwt = (dX && dW) ? L->dwt : nullptr;
        SNACK_CHECK(spmm_backward_fused(L, xt, dyt, p, B, dX, dW, dwt, s, rm, step));
        if (dwt && !(step && step->done)) {
            L->dwt_for = dW;
            L->dwt_valid = true;
        }
    } else {
        // short keys: a pass of its own for each of dX and dW
        const bool wx = dX && wide_short(L, L->tr, p), ww = dW && wide_short(L, L->fwd, p);
        if (!wx && !ww && dX && dW && wide_dw_fused(L, p)) {
            // one column pass for dX and dW over all batch tiles; dW in column order stays for the SGD step
            SNACK_CHECK(spmm_backward_wide(L, xt, dyt, p, B, dX, dW, L->dwt, ws_dw_slabs(L, p), s));
            L->dwt_for = dW;
            L->dwt_valid = true;
        } else {
            if (wx) {
                ProfScope prof(KC_SPMM_DX, s);
                SNACK_CHECK(wide_spmm(L, L->tr, dyt, p, B, dX, s));
            } else if (dX) {
                SNACK_CHECK(spmm_backward_fused(L, xt, dyt, p, B, dX, nullptr, nullptr, s));
            }
            if (ww) {
                ProfScope prof(KC_SDDMM_DW, s);
                SNACK_CHECK(wide_sddmm(L, xt, dyt, p, dW, s));
            } else if (dW) {
                SNACK_CHECK(sddmm_dw_tiles(L, xt, dyt, p, dW, s));
            }
        }
    }
    return SNACK_OK;
}

}  // namespace

extern "C" snack_status snack_backward(snack_layer* L, const float* X, const float* dY, float* dX, float* dW,
                                       int32_t B, snack_stream stream)
{
    if (!L || !dY || B < 1) return SNACK_ERR_INVALID_ARG;
    if (B > kMaxBatch) return SNACK_ERR_UNSUPPORTED;
    if (dW && !X) return SNACK_ERR_INVALID_ARG;
    if (dW && ((uintptr_t)dW & 15) != 0) return SNACK_ERR_INVALID_ARG;   // 16-byte vector stores
    if (!dX && !dW) return SNACK_OK;
    return backward_impl(L, X, dY, dX, dW, B, as_stream(stream), nullptr);
}

namespace {

// snack_backward_sgd after its argument checks
snack_status backward_sgd_impl(snack_layer* L, const float* X, const float* dY, float* dX, float* dW, float lr,
                               int32_t B, hipStream_t s, bool x_ready, bool dy_ready)
{
    SgdStep step{lr, false, false};
    ++L->vals_version;
    SNACK_CHECK(backward_impl(L, X, dY, dX, dW, B, s, &step, x_ready, dy_ready));
    if (!step.done) {
        // the column pass did not take the step: as snack_sgd_step would
        const float* dwt = (L->dwt_valid && dW == L->dwt_for) ? L->dwt : nullptr;
        L->dwt_valid = false;
        return sgd_update(L, dW, dwt, lr, s);
    }
    L->dwt_valid = false;
    if (step.canon_done) return SNACK_OK;   // the row pass stepped the canonical values too
    return sgd_update_values(L, dW, lr, s);
}

}  // namespace

extern "C" snack_status snack_backward_sgd(snack_layer* L, const float* X, const float* dY, float* dX, float* dW,
                                           float lr, int32_t B, snack_stream stream)
{
    if (!L || !X || !dY || B < 1 || (!dW && L->nnz > 0)) return SNACK_ERR_INVALID_ARG;
    if (B > kMaxBatch) return SNACK_ERR_UNSUPPORTED;
    if (((uintptr_t)dW & 15) != 0) return SNACK_ERR_INVALID_ARG;
    return backward_sgd_impl(L, X, dY, dX, dW, lr, B, as_stream(stream), false, false);
}

extern "C" snack_status snack_train_step_mse(snack_layer* L, const float* X, const float* T, float* Y, float* dY,
                                             float* dX, float* dW, float scale, float lr, int32_t B,
                                             snack_stream stream)
{
    if (!L || !X || !T || !Y || !dY || B < 1 || (!dW && L->nnz > 0)) return SNACK_ERR_INVALID_ARG;
    if (B > kMaxBatch) return SNACK_ERR_UNSUPPORTED;
    if (((uintptr_t)dW & 15) != 0) return SNACK_ERR_INVALID_ARG;
    hipStream_t s = as_stream(stream);
    const BatchPlan p = plan_batch(B);
    MseFuse m{T, dY, nullptr, scale, false, false};
    bool x_ready = false;
    if (spmm_batch_major(L, p, true, false, false)) {
        SNACK_CHECK(spmm_forward(L, X, p, B, Y, s, true, &m));
    } else {
        const float* feat = X;
        if (p.bp > 1) {
            // one feature-major copy of X for the forward and the backward; the forward's last pass can
            // write dY's feature-major copy too, where the backward takes one
            SNACK_CHECK(ws_check(L, p));
            SNACK_CHECK(transpose_pad(X, ws_x(L), L->K, nullptr, nullptr, 0, B, p.bp, s));
            feat = ws_x(L);
            x_ready = true;
            if (!spmm_batch_major(L, p, false, dX != nullptr, true)) m.dYt = ws_dy(L, p);
        }
        SNACK_CHECK(spmm_forward(L, feat, p, B, Y, s, false, &m));
    }
    if (!m.done) SNACK_CHECK(mse_grad(Y, T, dY, (int64_t)B * L->M, scale, s));
    return backward_sgd_impl(L, X, dY, dX, dW, lr, B, s, x_ready, m.dyt_done);
}

namespace {

// the inference forward of one layer, with the bf16 copy remade first when the
// values changed since it was made
snack_status forward_infer_one(snack_layer* L, const float* X, float* Y, int32_t B, int32_t act, bool b16,
                               hipStream_t s)
{
    if (act != kActNone && act != kActGelu) return SNACK_ERR_INVALID_ARG;
    if (!infer_supported(L, B, b16)) return SNACK_ERR_UNSUPPORTED;
    if (b16 && L->b16_version != L->vals_version) SNACK_CHECK(pack_bf16(L, s));
    return spmm_forward_infer(L, X, Y, B, act, b16, s);
}

}  // namespace

extern "C" snack_status snack_forward_infer(snack_layer* L, const float* X, float* Y, int32_t B, int32_t act,
                                            int32_t bf16_values, snack_stream stream)
{
    if (!L || !X || !Y || B < 1) return SNACK_ERR_INVALID_ARG;
    if (B > kMaxBatch) return SNACK_ERR_UNSUPPORTED;
    return forward_infer_one(L, X, Y, B, act, bf16_values != 0, as_stream(stream));
}

extern "C" snack_status snack_forward_chain(snack_layer* const* layers, int32_t n, const int32_t* acts,
                                            const float* X, float* const* Y, int32_t B, int32_t bf16_values,
                                            snack_stream stream)
{
    if (!layers || n < 1 || !acts || !X || !Y || B < 1) return SNACK_ERR_INVALID_ARG;
    if (B > kMaxBatch) return SNACK_ERR_UNSUPPORTED;
    // every check before the first launch, so a refused chain launches nothing
    for (int32_t i = 0; i < n; ++i) {
        const snack_layer* L = layers[i];
        if (!L || !Y[i] || (acts[i] != kActNone && acts[i] != kActGelu)) return SNACK_ERR_INVALID_ARG;
        if (i > 0 && L->K != layers[i - 1]->M) return SNACK_ERR_INVALID_ARG;
        if (!infer_supported(L, B, bf16_values != 0)) return SNACK_ERR_UNSUPPORTED;
    }
    hipStream_t s = as_stream(stream);
    for (int32_t i = 0; i < n; ++i)
        SNACK_CHECK(forward_infer_one(layers[i], i == 0 ? X : Y[i - 1], Y[i], B, acts[i], bf16_values != 0, s));
    return SNACK_OK;
}

extern "C" snack_status snack_prune_regrow(snack_layer* L, int64_t n_drop, snack_stream stream)
{
    if (!L || n_drop < 0 || n_drop > L->nnz) return SNACK_ERR_INVALID_ARG;
    L->dwt_valid = false;
    ++L->vals_version;
    return snack::prune_regrow(L, n_drop, as_stream(stream));
}

extern "C" snack_status snack_prune_regrow_grad(snack_layer* L, int64_t n_drop, const float* X, const float* dY,
                                                int32_t B, snack_stream stream)
{
    if (!L || n_drop < 0 || n_drop > L->nnz) return SNACK_ERR_INVALID_ARG;
    if (n_drop > 0 && (!X || !dY || B < 1)) return SNACK_ERR_INVALID_ARG;
    if (B > kMaxBatch) return SNACK_ERR_UNSUPPORTED;
    L->dwt_valid = false;
    ++L->vals_version;
    return snack::prune_regrow_grad(L, n_drop, X, dY, B, as_stream(stream));
}

extern "C" snack_status snack_prune_regrow_rows(snack_layer* L, int64_t drop_num, int64_t drop_den, int32_t mode,
                                                const float* X, const float* dY, int32_t B, snack_stream stream)
{
    if (!L || drop_den < 1 || drop_den > 0x7FFFFFFFll || drop_num < 0 || drop_num > drop_den) return SNACK_ERR_INVALID_ARG;
    if (mode != SNACK_REGROW_RANDOM && mode != SNACK_REGROW_GRADIENT) return SNACK_ERR_INVALID_ARG;
    const bool gradient = mode == SNACK_REGROW_GRADIENT;
    if (gradient && drop_num > 0 && (!X || !dY || B < 1)) return SNACK_ERR_INVALID_ARG;
    if (gradient && B > kMaxBatch) return SNACK_ERR_UNSUPPORTED;
    L->dwt_valid = false;
    ++L->vals_version;
    return snack::prune_regrow_rows(L, drop_num, drop_den, gradient, X, dY, B, as_stream(stream));
}

extern "C" snack_status snack_layer_shape(const snack_layer* L, int32_t* M, int32_t* K)
{
    if (!L || !M || !K) return SNACK_ERR_INVALID_ARG;
    *M = L->M;
    *K = L->K;
    return SNACK_OK;
}

extern "C" snack_status snack_layer_nnz(const snack_layer* L, int64_t* nnz)
{
    if (!L || !nnz) return SNACK_ERR_INVALID_ARG;
    *nnz = L->nnz;
    return SNACK_OK;
}

extern "C" snack_status snack_layer_device_bytes(const snack_layer* L, int64_t* bytes)
{
    if (!L || !bytes) return SNACK_ERR_INVALID_ARG;
    *bytes = (int64_t)L->device_bytes;
    return SNACK_OK;
}

extern "C" snack_status snack_layer_values(snack_layer* L, float** dev_values)
{
    if (!L || !dev_values) return SNACK_ERR_INVALID_ARG;
    *dev_values = L->vals;
    return SNACK_OK;
}

extern "C" snack_status snack_layer_values_updated(snack_layer* L)
{
    if (!L) return SNACK_ERR_INVALID_ARG;
    L->vals_t_stale = true;
    L->dwt_valid = false;
    ++L->vals_version;
    return SNACK_OK;
}

extern "C" snack_status snack_layer_export(const snack_layer* L, int32_t* rows, int32_t* cols, float* vals,
                                           snack_stream stream)
{
    if (!L) return SNACK_ERR_INVALID_ARG;
    hipStream_t s = as_stream(stream);
    const size_t n4 = (size_t)L->nnz * 4;
    if (n4 == 0) return SNACK_OK;
    if (rows) SNACK_HIP(hipMemcpyAsync(rows, L->rows, n4, hipMemcpyDeviceToDevice, s));
    if (cols) SNACK_HIP(hipMemcpyAsync(cols, L->cols, n4, hipMemcpyDeviceToDevice, s));
    if (vals) SNACK_HIP(hipMemcpyAsync(vals, L->vals, n4, hipMemcpyDeviceToDevice, s));
    return SNACK_OK;
}

extern "C" snack_status snack_layer_export_index(snack_layer* L, int32_t* row_ptr, int32_t* perm,
                                                 int32_t* rows_t, int32_t* col_ptr, float* vals_t,
                                                 snack_stream stream)
{
    if (!L) return SNACK_ERR_INVALID_ARG;
    hipStream_t s = as_stream(stream);
    const size_t n4 = (size_t)L->nnz * 4;
    if (row_ptr) SNACK_HIP(hipMemcpyAsync(row_ptr, L->row_ptr, ((size_t)L->M + 1) * 4, hipMemcpyDeviceToDevice, s));
    if (col_ptr) SNACK_HIP(hipMemcpyAsync(col_ptr, L->col_ptr, ((size_t)L->K + 1) * 4, hipMemcpyDeviceToDevice, s));
    if (n4) {
        if (perm) SNACK_CHECK(invert_iperm(L, perm, s));
        if (rows_t) SNACK_HIP(hipMemcpyAsync(rows_t, L->rows_t, n4, hipMemcpyDeviceToDevice, s));
        if (vals_t) {
            if (L->vals_t_stale) SNACK_CHECK(refresh_vals_t(L, s));
            SNACK_HIP(hipMemcpyAsync(vals_t, L->vals_t, n4, hipMemcpyDeviceToDevice, s));
        }
    }
    return SNACK_OK;
}

extern "C" snack_status snack_layer_get_epoch(const snack_layer* L, uint64_t* epoch)
{
    if (!L || !epoch) return SNACK_ERR_INVALID_ARG;
    *epoch = L->epoch;
    return SNACK_OK;
}

extern "C" snack_status snack_layer_set_epoch(snack_layer* L, uint64_t epoch)
{
    if (!L) return SNACK_ERR_INVALID_ARG;
    L->epoch = epoch;
    return SNACK_OK;
}

extern "C" snack_status snack_sgd_step(snack_layer* L, const float* dW, float lr, snack_stream stream)
{
    if (!L || (!dW && L->nnz > 0)) return SNACK_ERR_INVALID_ARG;
    // the caller may have changed dW since the backward (clipping, scaling), so
    // the column-ordered copy is refreshed from the stepped values before the
    // next pass that reads it, never stepped with a column-order dW of its own
    L->dwt_valid = false;
    ++L->vals_version;
    return sgd_update(L, dW, nullptr, lr, as_stream(stream));
}

extern "C" snack_status snack_mse_grad(const float* Y, const float* T, float* dY, int64_t n, float scale,
                                       snack_stream stream)
{
    if (n < 0 || (n > 0 && (!Y || !T || !dY))) return SNACK_ERR_INVALID_ARG;
    return mse_grad(Y, T, dY, n, scale, as_stream(stream));
}

extern "C" snack_status snack_gelu_fwd(const float* X, float* Y, int64_t n, snack_stream stream)
{
    if (n < 0 || (n > 0 && (!X || !Y))) return SNACK_ERR_INVALID_ARG;
    return gelu_fwd(X, Y, n, as_stream(stream));
}

extern "C" snack_status snack_gelu_bwd(const float* X, const float* dY, float* dX, int64_t n, snack_stream stream)
{
    if (n < 0 || (n > 0 && (!X || !dY || !dX))) return SNACK_ERR_INVALID_ARG;
    return gelu_bwd(X, dY, dX, n, as_stream(stream));
}
