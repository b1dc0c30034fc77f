/*
 * snack.h -- C ABI of the MI355X (gfx950) truly sparse COO layer.
 *
 * The layer stores its weight W [M x K] (out_features x in_features) only as
 * the COO triple of its stored positions -- values, row indices, column
 * indices -- and never materialises W.  This follows the SNACK paper ("Beyond
 * Masked Sparsity: SNACK Enables Truly Sparse Neural Networks on GPU"),
 * Figure 1: the block is a drop-in nn.Linear, the forward runs directly on the
 * triple, the backward is a sparse outer product over supp(W), and DST adds or
 * drops connections in place.  The transposed index used by the input gradient
 * is the cached transpose with a permutation map of the "Padded-CSR" post
 * (section 7.2) and the CSC column of the SNACK paper's Table 7.
 *
 * Conventions shared by every entry point:
 *  - Activations are fp32, contiguous, row-major in the nn.Linear layout:
 *    X [B, K], Y and dY [B, M], dX [B, K].  No bias.
 *  - Pointers marked "device" must be device memory on the layer's device,
 *    "host" host memory.  Device memory passed in stays owned by the caller.
 *  - `stream` is a hipStream_t (NULL selects the null stream).  Compute entry
 *    points are asynchronous on that stream; calls on one layer are ordered by
 *    the stream they are issued on.  A layer is not thread-safe.
 *  - Every call returns a snack_status.  Host-side argument checks are
 *    synchronous and leave the layer unchanged.  A HIP launch or runtime error
 *    is returned as SNACK_ERR_HIP; asynchronous device faults surface at the
 *    next synchronising call.  No C++ exception crosses this interface.
 *  - Index type is int32: nnz, M and K must each be below 2^31.
 *  - Device memory is allocated only by snack_layer_create and
 *    snack_layer_reserve.  Forward, backward, the fused training calls and
 *    drop/regrow allocate nothing and never synchronise the device (drop/regrow
 *    may wait on its own stream, see there).  A batch B is accepted when
 *    1 <= B <= 2^20 (else SNACK_ERR_UNSUPPORTED) and B is covered by the
 *    layer's reserved workspace (else SNACK_ERR_WORKSPACE); a refused call
 *    launches nothing and leaves the layer unchanged.
 *  - Canonical slot order: stored positions sorted by linear position
 *    row*K + col (row-major: by row, then column), as the sorted COO with a row
 *    pointer of the "Padded-CSR" post, section 3.2.  Values and dW are always
 *    in this order.
 */
#ifndef SNACK_H
#define SNACK_H

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum snack_status {
    SNACK_OK = 0,
    SNACK_ERR_INVALID_ARG = 1,   /* null pointer, negative size, shape mismatch, bad count */
    SNACK_ERR_INDEX_RANGE = 2,   /* a row or column index outside the matrix */
    SNACK_ERR_DUPLICATE = 3,     /* two entries name the same position */
    SNACK_ERR_ALLOC = 4,         /* device allocation failed */
    SNACK_ERR_HIP = 5,           /* a HIP runtime or launch error */
    SNACK_ERR_UNSUPPORTED = 6,   /* sizes beyond the int32 index range, or a batch above 2^20 */
    SNACK_ERR_WORKSPACE = 7      /* the batch needs more workspace than is reserved (snack_layer_reserve) */
} snack_status;

typedef struct snack_layer snack_layer;
typedef void* snack_stream;     /* hipStream_t */

/* Human-readable name of a status code (static storage, never NULL). */
const char* snack_status_string(snack_status s);

/*
 * Create a layer from an arbitrary-order COO triple.  SNACK paper, Figure 1
 * (the weight is the triple over the non-zeros) and "Padded-CSR" section 3.2
 * (sorted COO + row pointer).
 *   M, K        out_features, in_features (>= 1).
 *   nnz         number of stored positions (>= 0, <= M*K).
 *   rows, cols  device int32[nnz]; 0 <= rows < M, 0 <= cols < K; positions
 *               distinct (the support is a set).
 *   vals        device float[nnz], or NULL for all-zero values.
 *   seed        keys the regrow candidate stream; the epoch starts at 0.
 * The layer copies the triple (the caller may free its buffers on return),
 * sorts it into canonical order, builds the row pointer, the transposed index
 * and its work partition, reserves the per-batch workspace for every batch up
 * to 64 (as snack_layer_reserve(layer, 64)), and synchronises `stream` once to
 * report SNACK_ERR_INDEX_RANGE / SNACK_ERR_DUPLICATE.  On error *out is set to
 * NULL.
 */
snack_status snack_layer_create(int32_t M, int32_t K, int64_t nnz,
                                const int32_t* rows, const int32_t* cols, const float* vals,
                                uint64_t seed, snack_stream stream, snack_layer** out);

/* Free every buffer of the layer (synchronises the device first).  NULL is a no-op. */
snack_status snack_layer_destroy(snack_layer* layer);

/*
 * Size the per-batch workspace (feature-major copies of X and dY, and the
 * partial sums of the batch-tiled passes) for every batch up to max_batch
 * (1 <= max_batch <= 2^20, else SNACK_ERR_INVALID_ARG / SNACK_ERR_UNSUPPORTED).
 * The workspace never shrinks: a max_batch below the current reserve changes
 * nothing.  Growing it allocates the new workspace, synchronises the device
 * and frees the old one (SNACK_ERR_ALLOC when the allocation fails; the old
 * reserve then stays as it was).
 * Compute calls whose batch the reserve does not cover return
 * SNACK_ERR_WORKSPACE.
 */
snack_status snack_layer_reserve(snack_layer* layer, int32_t max_batch);

/*
 * Forward Y = X W^T.  SNACK paper, Figure 1 (forward on the triple, drop-in
 * nn.Linear); "Padded-CSR" section 6.1 (each live entry scales one input value
 * into its output row).
 *   X  device float[B, K];  Y device float[B, M], overwritten (rows of W with no
 *   stored position give 0).  1 <= B.  X and Y must not overlap.
 */
snack_status snack_forward(snack_layer* layer, const float* X, float* Y, int32_t B, snack_stream stream);

/*
 * Forward for callers that cannot allocate device memory (code under stream
 * capture, tight serving loops, harnesses that forbid allocation): the same
 * results, bit for bit, as snack_forward, with the scratch the forward needs
 * (the feature-major copy of X and the slice partial sums of the batch-tiled
 * pass) taken from one static device array of 48 MiB per device instead of
 * the layer's workspace; the call never allocates and needs no
 * snack_layer_reserve.  Plans needing more scratch than that array holds
 * return SNACK_ERR_WORKSPACE (at 10000 x 10000 and 95 % the limit admits
 * every batch up to 64).  The array is shared by every call on a device and
 * holds the last call's contents: calls that overlap on one device (two
 * streams, two threads) race and must be serialised by the caller.
 */
snack_status snack_forward_noalloc(snack_layer* layer, const float* X, float* Y, int32_t B, snack_stream stream);

/*
 * Inference forward: Y = act(X W^T) for batches up to 4 whose operand fits in
 * LDS (SNACK paper, Table 6: single-stream inference at batch 1 on the truly
 * sparse layer; "Padded-CSR" section 9.3: narrower index and value streams).
 * The streamed kernel reads 16-bit column indices (layers with in_features
 * below 65535) and either the fp32 values (6 bytes per entry) or, with
 * bf16_values, a copy of them rounded to bf16, nearest even (4 bytes per
 * entry); sums are fp32.  The copy is remade by the call itself whenever the
 * values changed since it was made (training calls, drop/regrow,
 * snack_layer_values_updated).  act: 0 none, 1 the exact GELU of
 * snack_gelu_fwd, applied to each output as it is stored.  With
 * bf16_values = 0 and act = 0 the result equals snack_forward bit for bit.
 *   X device float[B, K], Y device float[B, M] (overwritten).
 *   SNACK_ERR_UNSUPPORTED where the conditions above do not hold.
 */
snack_status snack_forward_infer(snack_layer* layer, const float* X, float* Y, int32_t B, int32_t act,
                                 int32_t bf16_values, snack_stream stream);

/*
 * A stack of layers run forward back to back, as snack_forward_infer each:
 * Y[0] = act[0](X W_0^T), Y[i] = act[i](Y[i-1] W_i^T).  layers, acts and Y are
 * host arrays of n entries; Y[i] is a device float[B, M_i]; the in_features of
 * layer i must equal the out_features of layer i-1.  Every argument is checked
 * before anything is launched.  The call allocates nothing and never
 * synchronises, so a caller may capture it in a HIP graph and replay it.
 */
snack_status snack_forward_chain(snack_layer* const* layers, int32_t n, const int32_t* acts, const float* X,
                                 float* const* Y, int32_t B, int32_t bf16_values, snack_stream stream);

/*
 * Backward.  "Padded-CSR" section 7.1: dX = dY W (the SpMM with the transpose,
 * run over the cached transposed index of section 7.2) and dW restricted to the
 * stored positions, dW[k] = sum_b dY[b, r_k] X[b, c_k]; the SNACK paper's
 * Figure 1 calls the latter the sparse outer product over supp(W).
 *   X   device float[B, K] (the forward's input), dY device float[B, M].
 *   dX  device float[B, K] or NULL (skipped); overwritten.
 *   dW  device float[nnz] in canonical slot order, 16-byte aligned, or NULL;
 *       overwritten (the caller accumulates if it wants to).  Stored zeros get
 *       a gradient.
 */
snack_status snack_backward(snack_layer* layer, const float* X, const float* dY,
                            float* dX, float* dW, int32_t B, snack_stream stream);

/*
 * Backward and the plain SGD step of the training loop in the "Padded-CSR"
 * post's section 8.2 ("Try It": loss.backward() then opt.step() of
 * torch.optim.SGD, i.e. each value moves against its gradient) in one call: the same results, bit
 * for bit, as snack_backward(layer, X, dY, dX, dW, B) followed by
 * snack_sgd_step(layer, dW, lr).  X, dY, dW are required (dW written as by
 * snack_backward; NULL only for a layer with no entries); dX may be NULL.  Where the column pass computes dW, it also
 * steps the layer's column-ordered value copy in place, so the step moves one
 * copy's worth of bytes less than the two separate calls.
 */
snack_status snack_backward_sgd(snack_layer* layer, const float* X, const float* dY, float* dX, float* dW,
                                float lr, int32_t B, snack_stream stream);

/*
 * One iteration of the training loop in the "Padded-CSR" post's section 8.2
 * ("Try It": forward, loss.backward(), opt.step() of plain SGD), in one call:
 * forward, loss gradient, backward and SGD step.  The loss is the mean squared
 * error against targets T; the pages' loop uses model(x).sum() instead, so the
 * MSE is this library's choice for training benchmarks, not the pages'.  The
 * same results, bit for bit, as
 *   snack_forward(layer, X, Y, B);
 *   snack_mse_grad(Y, T, dY, B * M, scale);
 *   snack_backward_sgd(layer, X, dY, dX, dW, lr, B);
 * (scale = 2 / (B * M) for the mean).  X device float[B, K]; T device
 * float[B, M] (the targets); Y, dY device float[B, M], overwritten; dX device
 * float[B, K] or NULL; dW device float[nnz], 16-byte aligned, overwritten (NULL
 * only for a layer with no entries).  The
 * forward's last pass writes dY beside Y (and the feature-major copy the
 * backward reads), and X is copied to feature-major order once for both
 * passes, so the call launches fewer passes than the three separate ones.
 */
snack_status snack_train_step_mse(snack_layer* layer, const float* X, const float* T, float* Y, float* dY,
                                  float* dX, float* dW, float scale, float lr, int32_t B, snack_stream stream);

/*
 * In-place drop / regrow with nnz fixed ("Padded-CSR" section 4.3: drop some
 * live entries, grow the same number elsewhere; SNACK paper Figure 1: in place
 * on the triple).  Drops the n_drop entries of smallest |value| -- order key
 * (IEEE bits of |v|, canonical slot), so -0 ties +0 and NaN is dropped last --
 * then grows n_drop positions uniformly at random among the positions empty
 * after the drop, with value +0.0: candidate t of epoch e is SplitMix64 output
 * number e*2^40 + t of the generator seeded with the layer's seed, mapped onto
 * [0, M*K) by the high word of the 64x64-bit product; a candidate is accepted
 * if its position is neither kept nor accepted earlier in the stream.  The
 * triple is re-canonicalised and the epoch incremented.  0 <= n_drop <= nnz.
 * May synchronise `stream` (once per candidate batch, normally once).  The
 * candidates are grouped by region in buckets of a fixed capacity; a batch
 * whose bucket overflows is taken again at half size, which does not change
 * the result.  For tests of that path, the environment variable
 * SNACK_GROW_BUCKET_CAP (a positive integer, read when a layer is created)
 * lowers the capacity of that layer's buckets.
 */
snack_status snack_prune_regrow(snack_layer* layer, int64_t n_drop, snack_stream stream);

/*
 * Drop / regrow with the regrow driven by the gradient (RigL-style): the
 * "Padded-CSR" post (section 4.3) has RigL drop a fraction of the live entries
 * and grow the same number "at high-gradient locations"; the SNACK paper
 * (Tables 8-9) trains with RigL on the truly sparse layer.  Drops the n_drop
 * entries of smallest |value| exactly as snack_prune_regrow, then grows n_drop
 * entries (value +0.0) at the cells empty after the drop whose dense weight
 * gradient for the batch (X, dY) is largest in magnitude:
 *   g[r, c] = sum over b of dY[b, r] X[b, c]   ("Padded-CSR" 7.1: dL/dW = dY^T X)
 * accumulated in fp32 with one fused multiply-add per batch row in batch
 * order; order key the IEEE bits of |g| (a NaN counts as 0), larger first,
 * ties by smaller linear position r*K + c.  No M*K array is stored: the
 * scores are recomputed by five sweeps over the cells (about 6 B M K flops
 * each).  The triple is re-canonicalised and the epoch incremented (the
 * random stream of snack_prune_regrow is not used).
 *   X   device float[B, K], dY device float[B, M]: batch-major (e.g. the last
 *       backward's input and output gradient); 1 <= B <= 2^20.
 *   0 <= n_drop <= nnz; requires M * K < 2^32 (else SNACK_ERR_UNSUPPORTED).
 */
snack_status snack_prune_regrow_grad(snack_layer* layer, int64_t n_drop, const float* X, const float* dY,
                                     int32_t B, snack_stream stream);

/*
 * Row-local drop / regrow: every row keeps its number of entries.  The
 * "Padded-CSR" post (section 8.3) notes that SparseLab's SET and RigL keep
 * per-row nnz fixed (only adaptive-density variants change it), so both the
 * drop and the regrow happen inside each row.  Row i with n_i entries drops
 * d_i = floor(n_i * drop_num / drop_den) of them -- its smallest |value|,
 * order key (IEEE bits of |v|, canonical slot) -- and grows d_i cells of the
 * same row that are empty after its drop, value +0.0:
 *   SNACK_REGROW_RANDOM (SET): candidate t of row i is the column
 *     high64(u_t * K), u_t = mix(s_i + (t + 1) * 0x9E3779B97F4A7C15) with
 *     s_i = mix(seed ^ mix(epoch * 2^32 + i)) and mix the SplitMix64 output
 *     function; a candidate is accepted if its cell is neither kept nor
 *     accepted at a smaller t.  Candidates t < 64 K + 4096 are tried; grows
 *     still missing after them (practically never) take the row's smallest
 *     empty columns.  X, dY and B are ignored.
 *   SNACK_REGROW_GRADIENT (RigL): the d_i empty cells of the row of largest
 *     |g|, g[i, c] = sum over b of dY[b, i] X[b, c] (the dense weight
 *     gradient, "Padded-CSR" 7.1), fp32 with one fused multiply-add per batch
 *     row in batch order, a NaN counting as 0; ties by smaller column.
 *     X device float[B, K], dY device float[B, M], batch-major, 1 <= B <= 2^20.
 * 0 <= drop_num <= drop_den, 1 <= drop_den <= 2^31 - 1.  The triple is
 * re-canonicalised and the epoch incremented (also when nothing moves).
 * Needs about 8 * (K / 32 + 130) bytes of LDS per row processed at once:
 * K up to about 650 000 (else SNACK_ERR_UNSUPPORTED).  Never synchronises.
 */
#define SNACK_REGROW_RANDOM 0
#define SNACK_REGROW_GRADIENT 1
snack_status snack_prune_regrow_rows(snack_layer* layer, int64_t drop_num, int64_t drop_den, int32_t mode,
                                     const float* X, const float* dY, int32_t B, snack_stream stream);

/* Shape and size queries (host outputs). */
snack_status snack_layer_shape(const snack_layer* layer, int32_t* M, int32_t* K);
snack_status snack_layer_nnz(const snack_layer* layer, int64_t* nnz);
/* Total bytes the layer holds in device memory (its own allocations). */
snack_status snack_layer_device_bytes(const snack_layer* layer, int64_t* bytes);

/*
 * Layer-owned device pointer to the canonical values (float[nnz]).  Valid until
 * destroy; prune_regrow rewrites its contents in place.  The caller may update
 * the values through it (an optimiser step) and must then call
 * snack_layer_values_updated before the next backward.
 */
snack_status snack_layer_values(snack_layer* layer, float** dev_values);
snack_status snack_layer_values_updated(snack_layer* layer);

/* Copy the canonical triple into caller device buffers (checkpointing, parity). */
snack_status snack_layer_export(const snack_layer* layer, int32_t* rows, int32_t* cols, float* vals,
                                snack_stream stream);

/*
 * Copy the index structures into caller device buffers ("Padded-CSR" 3.2 and
 * 7.2; SNACK Table 7): row_ptr int32[M+1], perm int32[nnz] (transposed slot ->
 * canonical slot), rows_t int32[nnz] (row of each transposed slot), col_ptr
 * int32[K+1], vals_t float[nnz] (the values in transposed order, equal to
 * vals[perm]).  Any pointer may be NULL.
 */
snack_status snack_layer_export_index(snack_layer* layer, int32_t* row_ptr, int32_t* perm,
                                      int32_t* rows_t, int32_t* col_ptr, float* vals_t, snack_stream stream);

/* Epoch = number of prune_regrow calls so far (resume: create + set_epoch). */
snack_status snack_layer_get_epoch(const snack_layer* layer, uint64_t* epoch);
snack_status snack_layer_set_epoch(snack_layer* layer, uint64_t epoch);

/*
 * Training-loop helpers (elementwise fp32; not part of the sparse method).
 *   snack_sgd_step:  values[k] -= lr * dW[k]   (dW device float[nnz], canonical order;
 *                    dW may be any array, e.g. a gradient the caller clipped
 *                    or scaled after snack_backward; the layer's column-ordered
 *                    value copy is rebuilt from the stepped values before the
 *                    next pass that reads it)
 *   snack_mse_grad:  dY[i] = scale * (Y[i] - T[i]), i < n   (MSE mean: scale = 2/n)
 *   snack_gelu_fwd:  Y = 0.5 X (1 + erf(X / sqrt 2))
 *   snack_gelu_bwd:  dX = dY * (Phi(X) + X phi(X))
 */
snack_status snack_sgd_step(snack_layer* layer, const float* dW, float lr, snack_stream stream);
snack_status snack_mse_grad(const float* Y, const float* T, float* dY, int64_t n, float scale,
                            snack_stream stream);
snack_status snack_gelu_fwd(const float* X, float* Y, int64_t n, snack_stream stream);
snack_status snack_gelu_bwd(const float* X, const float* dY, float* dX, int64_t n, snack_stream stream);

/*
 * Kernel timing.  While enabled, the library brackets each of its kernel
 * launches with HIP events recorded on the launch stream; snack_profile_read
 * synchronises those events and returns, for one kernel class, the launch count
 * and the summed duration in milliseconds.  Classes are numbered from 0;
 * snack_profile_name returns NULL past the last one.
 */
snack_status snack_profile_enable(int on);
snack_status snack_profile_reset(void);
const char* snack_profile_name(int kernel_class);
snack_status snack_profile_read(int kernel_class, int64_t* launches, double* total_ms);
/*
 * Tagged timing: launches made after snack_profile_set_tag(t) are also counted
 * under (kernel_class, t); snack_profile_read_tag returns those totals.  Tags
 * are caller-chosen integers (for example the batch size); at most 1024
 * distinct tags are kept.
 */
snack_status snack_profile_set_tag(int64_t tag);
snack_status snack_profile_read_tag(int kernel_class, int64_t tag, int64_t* launches, double* total_ms);

#ifdef __cplusplus
}
#endif

#endif /* SNACK_H */
