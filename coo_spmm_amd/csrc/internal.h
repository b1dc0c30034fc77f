// internal.h -- shared declarations of the HIP implementation of snack.h.
// Host code only sees launchers; every __global__ kernel lives in the .hip file
// that launches it.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>
#include <stddef.h>
#include <vector>

#include "../../include/snack.h"

namespace snack {

constexpr int kWave = 64;              // CDNA wavefront width
constexpr int kChunkWork = 512;        // most work (entries + keys) per SpMM chunk
constexpr int kChunkWorkMin = 128;     // least, for layers too small to fill the GPU with the most
constexpr int kChunkTarget = 1024;     // chunks per view a layer is cut into at least, where it can
constexpr int kPad = 2048;             // slack elements after every nnz-sized array
constexpr int32_t kMaxBatch = 1 << 20; // largest batch a call accepts
constexpr int32_t kDefaultReserve = 64; // batches a layer's workspace covers from create on
constexpr int32_t kIdx16Max = 65534;   // largest nidx whose indices (and the zero row past them) fit 16 bits

// Kernel classes for the profiling hooks (order = snack_profile_name ids).
enum KernelClass : int {
    KC_SPMM_FWD = 0,
    KC_SPMM_DX,
    KC_SDDMM_DW,
    KC_TRANSPOSE,
    KC_VALS_T_REFRESH,
    KC_SGD,
    KC_ELEMENTWISE,
    KC_SORT,
    KC_CANON,
    KC_PRUNE,
    KC_COUNT
};

// For the slice-tiled kernels: the gathered operand's rows split into S
// slices that each fit in LDS; tab[s * nkeys + r] is the first entry of key r
// whose index lies in slice s or later (s = 0..S).  Rebuilt lazily after every
// change of the index.
constexpr int kTileWidths = 4;   // batch tiles 8, 16, 32, 64
// Floats per staged row of the slice-tiled passes: a batch tile's columns,
// padded by 16 bytes below 64 columns so that consecutive rows start in
// different LDS banks (a lane group reads part of a row; at 64 columns each
// group reads whole 256-byte rows and needs no padding).
__host__ __device__ constexpr int tile_row_floats(int btile) { return btile < 64 ? btile + 4 : btile; }
constexpr int kMaxSplits = 64;   // most slices of one table
// one SGD step on one value: v - lr * g with a single rounding; every update of
// either value copy goes through it, so the two copies stay bit-identical
__device__ inline float sgd_value(float v, float g, float lr) { return fmaf(-lr, g, v); }
// exact (erf) GELU of one value: every kernel that applies it goes through this
__device__ inline float gelu_value(float x) { return 0.5f * x * (1.0f + erff(x * 0.70710678118654752f)); }
// activation codes of the inference forward
constexpr int kActNone = 0, kActGelu = 1;

// first index of slice s when [0, nidx) is cut into S slices
__host__ __device__ inline int32_t split_start(int32_t s, int32_t S, int32_t nidx)
{
    return (int32_t)(((int64_t)s * nidx) / S);
}
struct SplitTab {
    int32_t S = 0;
    int32_t* tab = nullptr;
    mutable bool valid = false;
};

// One sorted view of the triple: keys ascending (rows for the canonical view,
// cols for the transposed one), the gathered index, the values, the key
// pointer [nkeys+1] and the work partition into key-aligned chunks.
struct View {
    int32_t nkeys = 0;      // M (canonical) or K (transposed)
    int32_t nidx = 0;       // K (canonical) or M (transposed)
    int32_t* idx = nullptr;
    uint16_t* idx16 = nullptr;      // the same indices in 16 bits, where nidx < 65535 (else null)
    float* vals = nullptr;
    int32_t* ptr = nullptr;         // [nkeys + 1]
    int32_t nchunks = 0;
    int2* desc = nullptr;           // [nchunks + 1]: (first key, first entry) of each chunk
    int32_t* empty_keys = nullptr;  // [nkeys]: keys with no entry, ascending
    int32_t* n_empty = nullptr;     // device count of empty_keys
    SplitTab split[kTileWidths];
};

struct Scratch {
    size_t bytes = 0;
    void* base = nullptr;
};

}  // namespace snack

struct snack_layer {
    int device = 0;
    int lds_bytes = 0;   // LDS a workgroup may allocate on that device
    int cus = 0;         // compute units of that device
    int32_t M = 0, K = 0;
    int64_t nnz = 0;
    int64_t cap = 0;          // element capacity of each nnz-sized array (>= nnz + kPad)
    int32_t chunk_work = 0;   // work units per SpMM chunk (kChunkWorkMin .. kChunkWork)
    uint64_t seed = 0;
    uint64_t epoch = 0;
    int32_t grow_cap_max = 0;   // > 0: limit on the grow step's per-region buckets (retry-path tests)

    // canonical (row-sorted) triple
    int32_t* rows = nullptr;
    int32_t* cols = nullptr;
    float* vals = nullptr;
    int32_t* row_ptr = nullptr;   // [M+1]
    // transposed (column-sorted) index
    int32_t* iperm = nullptr;     // canonical slot -> transposed slot
    int32_t* rows_t = nullptr;
    float* vals_t = nullptr;      // values in transposed order
    // bf16 copy of the canonical values for the inference forward (round to
    // nearest even), remade when vals_version has moved past b16_version
    uint16_t* vals16 = nullptr;
    uint64_t vals_version = 1;
    uint64_t b16_version = 0;
    int32_t* col_ptr = nullptr;   // [K+1]
    bool vals_t_stale = true;
    // dW in transposed order from the last backward (bit-identical to the
    // canonical dW it was produced with); lets SGD update both value copies
    float* dwt = nullptr;
    const float* dwt_for = nullptr;
    bool dwt_valid = false;

    snack::View fwd;   // idx = cols
    snack::View tr;    // idx = rows_t

    // per-batch workspace: feature-major copies of X and dY
    float* ws = nullptr;
    size_t ws_bytes = 0;

    // scratch for sorting / prune_regrow (reserved at create)
    void* scratch = nullptr;
    size_t scratch_bytes = 0;
    int32_t* flag = nullptr;      // device error / count word(s)
    uint32_t* host_res = nullptr; // coherent pinned words the drop/regrow's grow result is written into
    uint32_t* host_res_dev = nullptr; // the same words as the device addresses them
    hipEvent_t grow_ev = nullptr; // recorded after that copy

    size_t device_bytes = 0;
    std::vector<void*> allocations;
};

namespace snack {

// ---- error handling ------------------------------------------------------
// With SNACK_DEBUG set in the environment, a failing HIP call is reported on
// stderr (expression, file, line, HIP's message) before the status returns.
void report_hip_error(hipError_t e, const char* expr, const char* file, int line);

#define SNACK_HIP(call)                                                   \
    do {                                                                  \
        hipError_t _e = (call);                                           \
        if (_e != hipSuccess) {                                           \
            ::snack::report_hip_error(_e, #call, __FILE__, __LINE__);     \
            return SNACK_ERR_HIP;                                         \
        }                                                                 \
    } while (0)

#define SNACK_CHECK(call)                                 \
    do {                                                  \
        snack_status _s = (call);                         \
        if (_s != SNACK_OK) return _s;                    \
    } while (0)

// ---- profiling hooks (prof.hip) ------------------------------------------
bool prof_on();
void prof_begin(int kclass, hipStream_t s);
void prof_end(int kclass, hipStream_t s);

struct ProfScope {
    int k;
    hipStream_t s;
    bool on;
    ProfScope(int kc, hipStream_t st) : k(kc), s(st), on(prof_on()) {
        if (on) prof_begin(k, s);
    }
    ~ProfScope() {
        if (on) prof_end(k, s);
    }
};

// ---- allocation helpers (layer.hip) ---------------------------------------
snack_status layer_alloc(snack_layer* L, void** p, size_t bytes);

// ---- sort / scan primitives (sort.hip) --------------------------------------
// Bytes of scratch needed to sort n (key, value) pairs with the given key width.
size_t radix_sort_scratch_bytes(int64_t n, int key_bits);
// Stable LSD radix sort of (keys, vals) by the low `key_bits` bits of keys.
// keys/vals are sorted in place; scratch must hold radix_sort_scratch_bytes.
snack_status radix_sort_u32(uint32_t* keys, uint32_t* vals, int64_t n, int key_bits, void* scratch,
                            hipStream_t s);
snack_status radix_sort_u64(uint64_t* keys, uint32_t* vals, int64_t n, int key_bits, void* scratch,
                            hipStream_t s);
// Exclusive prefix sum of int32 flags/counts (n elements), total written to *total_dev
// if non-null.  Scratch: scan_scratch_bytes(n).
size_t scan_scratch_bytes(int64_t n);
snack_status exclusive_scan_i32(const int32_t* in, int32_t* out, int64_t n, int32_t* total_dev, void* scratch,
                                hipStream_t s);

// ---- canonicalisation (canon.hip) -----------------------------------------
// Bytes of scratch canonicalise needs for nnz entries.
size_t canon_scratch_bytes(const snack_layer* L, int64_t nnz);
// Sort an arbitrary-order triple (device) into the layer's canonical arrays and
// validate it.  Writes error code into L->flag (0 ok).
snack_status canon_sort_input(snack_layer* L, const int32_t* rows, const int32_t* cols, const float* vals,
                              hipStream_t s);
// Given canonical rows/cols/vals, build row_ptr, the transposed view, vals_t,
// and both work partitions.
snack_status canon_build_index(snack_layer* L, hipStream_t s);
// The part of canon_build_index after row_ptr and the transposed view exist
// (for callers that build those themselves): partitions of both views, flags,
// and the 16-bit index copies unless the caller wrote them (idx16_done).
snack_status canon_index_tail(snack_layer* L, hipStream_t s, bool idx16_done = false, bool empty_cleared = false);
// vals_t[iperm[k]] = vals[k]
snack_status refresh_vals_t(snack_layer* L, hipStream_t s);
// the views' 16-bit index copies from their 32-bit indices (where allocated)
snack_status build_idx16(snack_layer* L, hipStream_t s);
// perm[iperm[k]] = k: the transposed slot -> canonical slot map, into a caller buffer
snack_status invert_iperm(const snack_layer* L, int32_t* perm, hipStream_t s);

// ---- kernels ---------------------------------------------------------------
// Batch tiling for a batch of B columns: B_tile columns per kernel pass, padded
// batch Bp (multiple of B_tile) used as the row stride of feature-major copies.
struct BatchPlan {
    int bt;      // lanes per group
    int nb;      // batch values per lane
    int u;       // run of entries per group per wave step
    int btile;   // bt * nb
    int bp;      // padded batch
    int ntiles;  // bp / btile
};
BatchPlan plan_batch(int B);

// dst[c * bp + b] = src[b * n + c] for b < B, 0 for B <= b < bp  (src [B, n]); the
// second pair (src2 may be null) is transposed by the same launch
snack_status transpose_pad(const float* src, float* dst, int n, const float* src2, float* dst2, int n2, int B,
                           int bp, hipStream_t s);

// Whether every kernel of a forward (fwd) or backward (dx, dw requested) pass
// can take the caller's batch-major [B][n] arrays directly, so no
// feature-major copy is needed (batch tiles up to 4, operands staged in LDS).
bool spmm_batch_major(const snack_layer* L, const BatchPlan& p, bool fwd, bool dx, bool dw);

// The MSE gradient of a forward's output written by the forward itself:
// dY = scale * (Y - T) (batch-major [B][M]) and, where dYt is set and the
// forward's last pass can, its feature-major copy [M][bp] (zero past B).
// done / dyt_done tell what the forward wrote.
struct MseFuse {
    const float* T;
    float* dY;
    float* dYt;
    float scale;
    bool done;
    bool dyt_done;
};

// Y[b, key] = sum over the canonical view's entries of v * Xt[idx, b]; with rm
// the operand is the batch-major X itself.  part: where the slice-tiled pass
// keeps its partial sums (forward_part_bytes of them); null selects the
// layer's workspace
snack_status spmm_forward(const snack_layer* L, const float* feat_t, const BatchPlan& p, int B, float* out,
                          hipStream_t s, bool rm = false, MseFuse* mse = nullptr, float* part = nullptr);
// Wide batches (more than one batch tile) over a view whose keys hold few
// entries (wide.hip): out[b, key] = sum of v * ft[idx, b] over the key's
// entries (ft feature-major [nidx][bp]), and dW[e] = sum_b dyt[r_e, b] xt[c_e, b]
bool wide_short(const snack_layer* L, const View& v, const BatchPlan& p);
snack_status wide_spmm(const snack_layer* L, const View& v, const float* ft, const BatchPlan& p, int B, float* out,
                       hipStream_t s);
snack_status wide_sddmm(const snack_layer* L, const float* xt, const float* dyt, const BatchPlan& p, float* dW,
                        hipStream_t s);
// bytes of slice partial sums the forward of plan p writes (0: none)
size_t forward_part_bytes(const snack_layer* L, const BatchPlan& p);

// one launch: dX over the transposed view (plus dW in transposed order when
// dW_t is non-null) and dW over the canonical view; either output may be null.
// Requires a single batch tile when dW or dW_t is requested.
// With `step`, where the column pass supports it, that pass also takes the SGD
// step vals_t -= lr * dW in place (from the values it loads) and step->done is
// set; dW_t is then written only where the canonical dW is permuted from it.
// Where the canonical dW comes from its own pass over the row view, that pass
// also steps vals in place and step->canon_done is set.
struct SgdStep {
    float lr;
    bool done;         // vals_t stepped
    bool canon_done;   // vals stepped
};
snack_status spmm_backward_fused(const snack_layer* L, const float* xt, const float* dyt, const BatchPlan& p, int B,
                                 float* dX, float* dW, float* dW_t, hipStream_t s, bool rm = false,
                                 SgdStep* step = nullptr);

// slice-tiled SpMM support: slices of view v for a batch tile (0 = not used),
// the split tables' allocation (at create) and the workspace the partial sums
// need for a batch plan
int tile_splits(const snack_layer* L, const View& v, int btile);
snack_status alloc_split_tables(snack_layer* L);
size_t tile_part_bytes(const snack_layer* L, const BatchPlan& p);
// several 64-column batch tiles: dX and dW in one slice-tiled column pass (one dW slab per tile,
// added up in tile order into dW_t, then permuted into canonical order into dW)
bool wide_dw_fused(const snack_layer* L, const BatchPlan& p);
size_t wide_dw_bytes(const snack_layer* L, const BatchPlan& p);   // the slabs; 0 where not taken
snack_status spmm_backward_wide(const snack_layer* L, const float* xt, const float* dyt, const BatchPlan& p, int B,
                                float* dX, float* dW, float* dW_t, float* slabs, hipStream_t s);
float* ws_part(const snack_layer* L, const BatchPlan& p);   // layer.hip

// dW for batches wider than one tile (loops over the tiles)
snack_status sddmm_dw_tiles(const snack_layer* L, const float* xt, const float* dyt, const BatchPlan& p, float* dW,
                            hipStream_t s);

// values -= lr * dW; also vals_t -= lr * dW_t when dW_t is non-null
snack_status sgd_update(snack_layer* L, const float* dW, const float* dW_t, float lr, hipStream_t s);
// values -= lr * dW only (vals_t already took the step in the column pass)
snack_status sgd_update_values(snack_layer* L, const float* dW, float lr, hipStream_t s);
snack_status mse_grad(const float* Y, const float* T, float* dY, int64_t n, float scale, hipStream_t s);
snack_status gelu_fwd(const float* X, float* Y, int64_t n, hipStream_t s);
// vals16 = the values rounded to bf16 (nearest even)
snack_status pack_bf16(snack_layer* L, hipStream_t s);
// the inference forward (batch tiles up to 4, operand in LDS): Y = act(X W^T), with
// the values from the bf16 copy when b16; SNACK_ERR_UNSUPPORTED where it does not apply
snack_status spmm_forward_infer(const snack_layer* L, const float* X, float* Y, int B, int act, bool b16,
                                hipStream_t s);
bool infer_supported(const snack_layer* L, int B, bool b16);
snack_status gelu_bwd(const float* X, const float* dY, float* dX, int64_t n, hipStream_t s);

// ---- prune / regrow (prune.hip) ---------------------------------------------
size_t prune_scratch_bytes(const snack_layer* L);
snack_status prune_regrow(snack_layer* L, int64_t n_drop, hipStream_t s);
// the same drop, then the regrow at the empty cells of largest |dL/dW| for the batch (X, dY)
// Row-local drop / regrow (rows.hip): the bitmaps and value copy that the
// rebuild of the global drop / regrow takes.
struct RowDst {
    const int32_t* row_ptr;
    const int32_t* cols;
    const float* vals;
    float* vcopy;
    uint32_t* old_bm;
    uint32_t* kept_bm;
    uint32_t* occ_bm;
    int32_t M, K;
    int64_t num, den;
    bool gradient;
    uint64_t seed, epoch;
    const float* X;
    const float* dY;
    int32_t B;
};
int64_t rows_lds_per_wave(int32_t K);
snack_status rows_drop_grow(const RowDst& r, int lds_limit, hipStream_t s);
snack_status prune_regrow_rows(snack_layer* L, int64_t num, int64_t den, bool gradient, const float* X,
                               const float* dY, int32_t B, hipStream_t s);
snack_status prune_regrow_grad(snack_layer* L, int64_t n_drop, const float* X, const float* dY, int32_t B,
                               hipStream_t s);

// ---- gradient regrow (rigl.hip) ----------------------------------------------
// Cells are scored in tiles of kGradTile x kGradTile; ties at the threshold are
// counted per row and column tile.
constexpr int kGradTile = 128;
constexpr int kGradHistWords = 2048 + 4096 + 256;
inline int64_t grad_col_tiles(int32_t K) { return ((int64_t)K + kGradTile - 1) / kGradTile; }
struct GradGrow {
    const uint32_t* kept_bm;   // cells kept by the drop (the grow picks among the others)
    uint32_t* occ_bm;          // written: the kept cells and the grown ones
    int64_t words;
    int64_t need;              // cells to grow
    const float* X;            // [B][K] batch-major
    const float* dY;           // [B][M] batch-major
    int32_t B;
    uint32_t* state;           // [16]
    uint32_t* hist;            // [kGradHistWords]
    int32_t* tie_cnt;          // [M * grad_col_tiles(K)]
    void* scan;                // scan scratch for M * grad_col_tiles(K) elements
};
snack_status grow_by_gradient(const snack_layer* L, const GradGrow& g, hipStream_t s);

}  // namespace snack
