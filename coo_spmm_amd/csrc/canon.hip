// canon.hip -- canonical order, validation and index structures of the layer.
//
// Canonical order: stored positions sorted by linear position row*K + col,
// i.e. by row then column -- the sorted COO with a row pointer of the
// "Padded-CSR" post, section 3.2.  The transposed view lists the same slots
// sorted by (column, row) together with the permutation map of section 7.2
// (transposed slot -> canonical slot) and the column pointer (the CSC of the
// SNACK paper's Table 7).  Both views carry a key-aligned work partition:
// desc[c] = (first key, first entry) of chunk c, cut so that each chunk holds
// about the layer's chunk_work units of (entries + keys); a key is never split, so the
// SpMM needs no cross-chunk fix-up and writes every output row once.  Each view
// also lists its keys without entries, whose outputs are zero.
#include "internal.h"

namespace snack {
namespace {

constexpr int kThreads = 256;

inline unsigned grid_for(int64_t n, int per_block = kThreads)
{
    int64_t g = (n + per_block - 1) / per_block;
    if (g < 1) g = 1;
    if (g > 65535LL * 16) g = 65535LL * 16;
    return (unsigned)g;
}

inline int bits_for(uint64_t maxval)
{
    int b = 1;
    while (b < 64 && (maxval >> b) != 0) ++b;
    return b;
}

// Linear position keys with range validation.  flag |= 1 on a bad index.
template <typename KeyT>
__global__ void make_keys_kernel(const int32_t* __restrict__ rows, const int32_t* __restrict__ cols, int64_t nnz,
                                 int32_t M, int32_t K, KeyT* __restrict__ keys, uint32_t* __restrict__ slots,
                                 int32_t* __restrict__ flag)
{
    for (int64_t k = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; k < nnz; k += (int64_t)gridDim.x * blockDim.x) {
        const int32_t r = rows[k], c = cols[k];
        KeyT key = 0;
        if (r < 0 || r >= M || c < 0 || c >= K) {
            atomicOr(flag, 1);
        } else {
            key = (KeyT)r * (KeyT)K + (KeyT)c;
        }
        keys[k] = key;
        slots[k] = (uint32_t)k;
    }
}

// Canonical arrays from the sorted keys; flag |= 2 on a repeated position.
template <typename KeyT>
__global__ void gather_canonical_kernel(const KeyT* __restrict__ keys, const uint32_t* __restrict__ slots,
                                        int64_t nnz, int32_t K, const float* __restrict__ vin,
                                        int32_t* __restrict__ rows, int32_t* __restrict__ cols,
                                        float* __restrict__ vals, int32_t* __restrict__ flag)
{
    for (int64_t k = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; k < nnz; k += (int64_t)gridDim.x * blockDim.x) {
        const KeyT key = keys[k];
        if (k > 0 && keys[k - 1] == key) atomicOr(flag, 2);
        rows[k] = (int32_t)(key / (KeyT)K);
        cols[k] = (int32_t)(key % (KeyT)K);
        vals[k] = vin ? vin[slots[k]] : 0.0f;
    }
}

// ptr[r] = first slot whose key >= r, for r in [0, nkeys]; keys sorted.
__global__ void build_ptr_kernel(const int32_t* __restrict__ keys, int64_t nnz, int32_t nkeys,
                                 int32_t* __restrict__ ptr)
{
    for (int64_t k = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; k <= nnz;
         k += (int64_t)gridDim.x * blockDim.x) {
        const int32_t prev = (k == 0) ? -1 : keys[k - 1];
        const int32_t cur = (k == nnz) ? nkeys : keys[k];
        for (int32_t r = prev + 1; r <= cur; ++r) ptr[r] = (int32_t)k;
    }
}

// desc[c] = (r, ptr[r]) with r the smallest key such that ptr[r] + r >= c * work;
// desc[nchunks] = (nkeys, nnz).  One launch serves both views (blockIdx.y);
// it also clears the views' empty-key counters for the append that follows.
struct PartArgs {
    const int32_t* ptr;
    int32_t nkeys;
    int32_t nchunks;
    int2* desc;
    int32_t* empty_keys;
    int32_t* n_empty;
};

__device__ inline void chunks_part(const PartArgs& v, int32_t work, int bx, int nbx)
{
    for (int64_t c = (int64_t)bx * blockDim.x + threadIdx.x; c <= v.nchunks; c += (int64_t)nbx * blockDim.x) {
        int32_t key = v.nkeys;
        if (c < v.nchunks) {
            const int64_t target = c * (int64_t)work;
            int32_t lo = 0, hi = v.nkeys;
            while (lo < hi) {
                const int32_t mid = lo + ((hi - lo) >> 1);
                if ((int64_t)v.ptr[mid] + mid >= target) hi = mid;
                else lo = mid + 1;
            }
            key = lo;
        }
        v.desc[c] = make_int2(key, v.ptr[key]);
    }
}

__global__ void build_chunks_kernel(PartArgs va, PartArgs vb, int32_t work)
{
    const PartArgs& v = blockIdx.y == 0 ? va : vb;
    if (blockIdx.x == 0 && threadIdx.x == 0) *v.n_empty = 0;
    chunks_part(v, work, (int)blockIdx.x, (int)gridDim.x);
}

// Keys without entries, in no particular order (the SpMM only writes zeros
// for them, so the order cannot change any result); one atomic per wave.
__device__ inline void empty_part(const PartArgs& v, int bx, int nbx)
{
    const int lane = threadIdx.x & (kWave - 1);
    const int64_t stride = (int64_t)nbx * blockDim.x;
    for (int64_t r0 = (int64_t)bx * blockDim.x; r0 < v.nkeys; r0 += stride) {
        const int64_t r = r0 + threadIdx.x;
        const bool empty = r < v.nkeys && v.ptr[r] == v.ptr[r + 1];
        const uint64_t m = __ballot(empty);
        if (m == 0) continue;
        int32_t base = 0;
        if (lane == __ffsll((unsigned long long)m) - 1) base = atomicAdd(v.n_empty, __popcll(m));
        base = __shfl(base, __ffsll((unsigned long long)m) - 1, kWave);
        if (empty) v.empty_keys[base + __popcll(m & ((1ull << lane) - 1ull))] = (int32_t)r;
    }
}

__global__ void empty_keys_kernel(PartArgs va, PartArgs vb)
{
    empty_part(blockIdx.y == 0 ? va : vb, (int)blockIdx.x, (int)gridDim.x);
}

// Both in one launch when the empty-key counters are already zero: of a grid
// row (one view), the first `nbc` workgroups build the chunk descriptors and
// the others list the empty keys.
__global__ void partition_kernel(PartArgs va, PartArgs vb, int32_t work, int32_t nbc)
{
    const PartArgs& v = blockIdx.y == 0 ? va : vb;
    if ((int)blockIdx.x < nbc) chunks_part(v, work, (int)blockIdx.x, nbc);
    else empty_part(v, (int)blockIdx.x - nbc, (int)gridDim.x - nbc);
}

__global__ void iota_cols_kernel(const int32_t* __restrict__ cols, int64_t nnz, uint32_t* __restrict__ keys,
                                 uint32_t* __restrict__ slots)
{
    for (int64_t k = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; k < nnz; k += (int64_t)gridDim.x * blockDim.x) {
        keys[k] = (uint32_t)cols[k];
        slots[k] = (uint32_t)k;
    }
}

__global__ void build_transposed_kernel(const uint32_t* __restrict__ tslots, int64_t nnz,
                                        const int32_t* __restrict__ rows, const float* __restrict__ vals,
                                        int32_t* __restrict__ iperm, int32_t* __restrict__ rows_t,
                                        float* __restrict__ vals_t)
{
    for (int64_t j = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; j < nnz; j += (int64_t)gridDim.x * blockDim.x) {
        const int32_t k = (int32_t)tslots[j];
        iperm[k] = (int32_t)j;
        rows_t[j] = rows[k];
        vals_t[j] = vals[k];
    }
}

// ---- transposed view by a stable counting sort on the column --------------
// The canonical slots are cut into nb contiguous ranges of E entries, one
// workgroup each.  tb_count writes the workgroup's column histogram into
// mat[c * nb + b]; an exclusive scan of mat in that (column-major) order gives
// every (column, range) pair its first transposed slot.  tb_scatter then walks
// its range in canonical order with one LDS cursor per column.  A row holds a
// column at most once, so the entries of one row never collide; rows are taken
// one after another (a barrier between them), which keeps each column's
// entries in row order without any sort and without global atomics.
// Workgroups are dispatched to the 8 XCDs round-robin; range b is given to the
// workgroup that puts ranges [x*per, (x+1)*per) on XCD x, so the slots of one
// column written from neighbouring ranges meet in the same L2 and leave it as
// whole lines.
constexpr int kTbThreads = 512;
constexpr int kXcds = 8;
constexpr int32_t kTbMaxKeys = 15360;            // cursor array of 60 KB in LDS
constexpr int64_t kTbMatrixMax = 4 << 20;        // nb * K

__global__ void __launch_bounds__(kTbThreads) tb_count_kernel(const int32_t* __restrict__ cols, int64_t nnz,
                                                              int64_t E, int32_t K, int32_t nb,
                                                              int32_t* __restrict__ mat)
{
    extern __shared__ int32_t hist[];
    const int32_t per = gridDim.x / kXcds;
    const int32_t b = (int32_t)(blockIdx.x % kXcds) * per + (int32_t)(blockIdx.x / kXcds);
    if (b >= nb) return;
    for (int32_t c = threadIdx.x; c < K; c += kTbThreads) hist[c] = 0;
    __syncthreads();
    const int64_t e0 = (int64_t)b * E;
    const int64_t e1 = e0 + E < nnz ? e0 + E : nnz;
    // eight loads in flight per thread; indexes clamped so every load is issued
    for (int64_t base = e0; base < e1; base += 8 * kTbThreads) {
        int32_t c[8];
#pragma unroll
        for (int u = 0; u < 8; ++u) {
            const int64_t k = base + u * kTbThreads + threadIdx.x;
            c[u] = cols[k < e1 ? k : e1 - 1];
        }
#pragma unroll
        for (int u = 0; u < 8; ++u)
            if (base + u * kTbThreads + threadIdx.x < e1) atomicAdd(&hist[c[u]], 1);
    }
    __syncthreads();
    for (int32_t c = threadIdx.x; c < K; c += kTbThreads) mat[(int64_t)c * nb + b] = hist[c];
}

// Loads run two rounds ahead, and every lane issues the same loads and stores
// (clamped reads; a lane past the range writes zeros into the zero padding
// after slot nnz), so the compiler's wait before a round covers that round's
// loads only, never the scattered stores of the rounds before it.
struct TbEntry {
    int32_t r, c;
    float v;
};

__global__ void __launch_bounds__(kTbThreads) tb_scatter_kernel(
    const int32_t* __restrict__ rows, const int32_t* __restrict__ cols, const float* __restrict__ vals, int64_t nnz,
    int64_t E, int32_t K, int32_t nb, const int32_t* __restrict__ mat, int32_t* __restrict__ iperm,
    int32_t* __restrict__ rows_t, float* __restrict__ vals_t,
    int32_t* __restrict__ col_ptr)
{
    extern __shared__ int32_t cur[];
    __shared__ int32_t s_row[kTbThreads];
    __shared__ int32_t s_wave[kTbThreads / kWave];
    const int32_t per = gridDim.x / kXcds;
    const int32_t b = (int32_t)(blockIdx.x % kXcds) * per + (int32_t)(blockIdx.x / kXcds);
    if (b >= nb) return;
    const int tid = threadIdx.x, lane = tid & (kWave - 1), w = tid / kWave;
    for (int32_t c = tid; c < K; c += kTbThreads) {
        const int32_t v = mat[(int64_t)c * nb + b];
        cur[c] = v;
        if (b == 0) col_ptr[c] = v;
    }
    if (b == 0 && tid == 0) col_ptr[K] = (int32_t)nnz;
    const int64_t e0 = (int64_t)b * E;
    const int64_t e1 = e0 + E < nnz ? e0 + E : nnz;
    if (e0 >= e1) return;   // uniform over the workgroup
    auto load = [&](int64_t k, TbEntry& x) {
        const int64_t kc = k < e1 ? k : e1 - 1;
        x.r = rows[kc];
        x.c = cols[kc];
        x.v = vals[kc];
    };
    auto round = [&](int64_t k, const TbEntry& x) {
        const bool live = k < e1;
        s_row[tid] = live ? x.r : -1;
        __syncthreads();
        const bool start = live && (tid == 0 || s_row[tid - 1] != x.r);
        const uint64_t m = __ballot(start);
        const int upto = __popcll(m & (lane == kWave - 1 ? ~0ull : ((2ull << lane) - 1ull)));
        if (lane == 0) s_wave[w] = __popcll(m);
        __syncthreads();
        int before = 0, nseg = 0;
#pragma unroll
        for (int i = 0; i < kTbThreads / kWave; ++i) {
            const int y = s_wave[i];
            before += i < w ? y : 0;
            nseg += y;
        }
        const int seg = before + upto - 1;
        int32_t pos = (int32_t)nnz + tid;
        for (int sg = 0; sg < nseg; ++sg) {
            if (live && seg == sg) {
                pos = cur[x.c];
                cur[x.c] = pos + 1;
            }
            __syncthreads();
        }
        rows_t[pos] = live ? x.r : 0;
        vals_t[pos] = live ? x.v : 0.0f;
        iperm[live ? k : nnz + tid] = live ? pos : 0;
    };
    TbEntry A, B;
    int64_t k = e0 + tid;
    load(k, A);
    load(k + kTbThreads, B);
    __syncthreads();
    for (; k - tid < e1; k += 2 * kTbThreads) {
        const TbEntry a = A;
        load(k + 2 * kTbThreads, A);
        round(k, a);
        if (k - tid + kTbThreads >= e1) break;   // uniform
        const TbEntry bb = B;
        load(k + 3 * kTbThreads, B);
        round(k + kTbThreads, bb);
    }
}

inline void tb_plan(int64_t nnz, int32_t K, int32_t* nb_out, int64_t* e_out)
{
    int64_t nb = (nnz + 4095) / 4096;
    const int64_t lim = kTbMatrixMax / (K > 0 ? K : 1);
    if (nb > lim) nb = lim;
    if (nb > 1024) nb = 1024;
    if (nb < 1) nb = 1;
    *nb_out = (int32_t)nb;
    *e_out = (nnz + nb - 1) / nb;
}

__global__ void refresh_vals_t_kernel(const int32_t* __restrict__ iperm, const float* __restrict__ vals, int64_t nnz,
                                      float* __restrict__ vals_t)
{
    for (int64_t k = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; k < nnz; k += (int64_t)gridDim.x * blockDim.x)
        vals_t[iperm[k]] = vals[k];
}

__global__ void invert_iperm_kernel(const int32_t* __restrict__ iperm, int64_t nnz, int32_t* __restrict__ perm)
{
    for (int64_t k = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; k < nnz; k += (int64_t)gridDim.x * blockDim.x)
        perm[iperm[k]] = (int32_t)k;
}

snack_status build_view_partitions(snack_layer* L, hipStream_t s, bool empty_cleared)
{
    auto args = [](const View& v) {
        PartArgs a;
        a.ptr = v.ptr;
        a.nkeys = v.nkeys;
        a.nchunks = v.nchunks;
        a.desc = v.desc;
        a.empty_keys = v.empty_keys;
        a.n_empty = v.n_empty;
        return a;
    };
    const PartArgs a = args(L->fwd), b = args(L->tr);
    const int32_t nc = a.nchunks > b.nchunks ? a.nchunks : b.nchunks;
    const int32_t nk = a.nkeys > b.nkeys ? a.nkeys : b.nkeys;
    if (empty_cleared) {
        const unsigned nbc = grid_for((int64_t)nc + 1), nbe = grid_for(nk);
        hipLaunchKernelGGL(partition_kernel, dim3(nbc + nbe, 2), dim3(kThreads), 0, s, a, b, L->chunk_work,
                           (int32_t)nbc);
    } else {
        hipLaunchKernelGGL(build_chunks_kernel, dim3(grid_for((int64_t)nc + 1), 2), dim3(kThreads), 0, s, a, b,
                           L->chunk_work);
        hipLaunchKernelGGL(empty_keys_kernel, dim3(grid_for(nk), 2), dim3(kThreads), 0, s, a, b);
    }
    SNACK_HIP(hipGetLastError());
    return SNACK_OK;
}

}  // namespace

size_t canon_scratch_bytes(const snack_layer* L, int64_t nnz)
{
    const uint64_t N = (uint64_t)L->M * (uint64_t)L->K;
    const int kb = bits_for(N > 0 ? N - 1 : 0);
    const size_t kw = kb > 32 ? 8 : 4;
    size_t b = 0;
    b += ((size_t)nnz * kw + 255) & ~(size_t)255;     // keys
    b += ((size_t)nnz * 4 + 255) & ~(size_t)255;      // slots
    b += radix_sort_scratch_bytes(nnz, kb);
    // empty-key lists of the two views
    const int64_t nk = L->M > L->K ? L->M : L->K;
    size_t e = 2 * (((size_t)nk + 63) & ~(size_t)63) * 4 + scan_scratch_bytes(nk) + 256;
    if (L->K <= kTbMaxKeys) {
        int32_t nb;
        int64_t E;
        tb_plan(nnz, L->K, &nb, &E);
        const size_t m = (size_t)nb * L->K;
        const size_t t = ((m * 4 + 255) & ~(size_t)255) + scan_scratch_bytes((int64_t)m);
        if (t > e) e = t;
    }
    return (b > e ? b : e) + 256;
}

snack_status canon_sort_input(snack_layer* L, const int32_t* rows, const int32_t* cols, const float* vals,
                              hipStream_t s)
{
    ProfScope prof(KC_CANON, s);
    const int64_t nnz = L->nnz;
    if (nnz == 0) return SNACK_OK;
    const uint64_t N = (uint64_t)L->M * (uint64_t)L->K;
    const int kb = bits_for(N - 1);
    char* p = (char*)L->scratch;
    if (kb > 32) {
        uint64_t* keys = (uint64_t*)p;
        p += ((size_t)nnz * 8 + 255) & ~(size_t)255;
        uint32_t* slots = (uint32_t*)p;
        p += ((size_t)nnz * 4 + 255) & ~(size_t)255;
        hipLaunchKernelGGL(make_keys_kernel<uint64_t>, dim3(grid_for(nnz)), dim3(kThreads), 0, s, rows, cols, nnz,
                           L->M, L->K, keys, slots, L->flag);
        SNACK_HIP(hipGetLastError());
        SNACK_CHECK(radix_sort_u64(keys, slots, nnz, kb, p, s));
        hipLaunchKernelGGL(gather_canonical_kernel<uint64_t>, dim3(grid_for(nnz)), dim3(kThreads), 0, s, keys, slots,
                           nnz, L->K, vals, L->rows, L->cols, L->vals, L->flag);
        SNACK_HIP(hipGetLastError());
    } else {
        uint32_t* keys = (uint32_t*)p;
        p += ((size_t)nnz * 4 + 255) & ~(size_t)255;
        uint32_t* slots = (uint32_t*)p;
        p += ((size_t)nnz * 4 + 255) & ~(size_t)255;
        hipLaunchKernelGGL(make_keys_kernel<uint32_t>, dim3(grid_for(nnz)), dim3(kThreads), 0, s, rows, cols, nnz,
                           L->M, L->K, keys, slots, L->flag);
        SNACK_HIP(hipGetLastError());
        SNACK_CHECK(radix_sort_u32(keys, slots, nnz, kb, p, s));
        hipLaunchKernelGGL(gather_canonical_kernel<uint32_t>, dim3(grid_for(nnz)), dim3(kThreads), 0, s, keys, slots,
                           nnz, L->K, vals, L->rows, L->cols, L->vals, L->flag);
        SNACK_HIP(hipGetLastError());
    }
    return SNACK_OK;
}

snack_status canon_build_index(snack_layer* L, hipStream_t s)
{
    ProfScope prof(KC_CANON, s);
    const int64_t nnz = L->nnz;
    hipLaunchKernelGGL(build_ptr_kernel, dim3(grid_for(nnz + 1)), dim3(kThreads), 0, s, L->rows, nnz, L->M,
                       L->row_ptr);
    SNACK_HIP(hipGetLastError());
    if (nnz > 0 && L->K <= kTbMaxKeys) {
        int32_t nb;
        int64_t E;
        tb_plan(nnz, L->K, &nb, &E);
        int32_t* mat = (int32_t*)L->scratch;
        const size_t m = (size_t)nb * L->K;
        void* scan_scr = (char*)L->scratch + ((m * 4 + 255) & ~(size_t)255);
        const size_t lds = (size_t)L->K * 4;
        const unsigned grid = (unsigned)((nb + kXcds - 1) / kXcds * kXcds);
        hipLaunchKernelGGL(tb_count_kernel, dim3(grid), dim3(kTbThreads), lds, s, L->cols, nnz, E, L->K, nb, mat);
        SNACK_HIP(hipGetLastError());
        SNACK_CHECK(exclusive_scan_i32(mat, mat, (int64_t)m, nullptr, scan_scr, s));
        hipLaunchKernelGGL(tb_scatter_kernel, dim3(grid), dim3(kTbThreads), lds, s, L->rows, L->cols, L->vals, nnz, E,
                           L->K, nb, mat, L->iperm, L->rows_t, L->vals_t, L->col_ptr);
        SNACK_HIP(hipGetLastError());
    } else {
        if (nnz > 0) {
            // many columns: stable radix sort of the slots by column instead
            char* p = (char*)L->scratch;
            uint32_t* tkeys = (uint32_t*)p;
            p += ((size_t)nnz * 4 + 255) & ~(size_t)255;
            uint32_t* tslots = (uint32_t*)p;
            p += ((size_t)nnz * 4 + 255) & ~(size_t)255;
            hipLaunchKernelGGL(iota_cols_kernel, dim3(grid_for(nnz)), dim3(kThreads), 0, s, L->cols, nnz, tkeys,
                               tslots);
            SNACK_HIP(hipGetLastError());
            // canonical order is (row, col), so a stable sort by column yields (col, row)
            SNACK_CHECK(radix_sort_u32(tkeys, tslots, nnz, bits_for((uint64_t)(L->K - 1)), p, s));
            hipLaunchKernelGGL(build_transposed_kernel, dim3(grid_for(nnz)), dim3(kThreads), 0, s, tslots, nnz,
                               L->rows, L->vals, L->iperm, L->rows_t, L->vals_t);
            // the sorted keys are the columns in transposed order
            hipLaunchKernelGGL(build_ptr_kernel, dim3(grid_for(nnz + 1)), dim3(kThreads), 0, s,
                               (const int32_t*)tkeys, nnz, L->K, L->col_ptr);
            SNACK_HIP(hipGetLastError());
        } else {
            hipLaunchKernelGGL(build_ptr_kernel, dim3(grid_for(1)), dim3(kThreads), 0, s, L->rows, (int64_t)0,
                               L->K, L->col_ptr);
            SNACK_HIP(hipGetLastError());
        }
    }
    return canon_index_tail(L, s);
}

// 16-bit copies of a view's indices: four per thread, the padding past nnz zero
__global__ void idx16_kernel(const int32_t* __restrict__ a, uint16_t* __restrict__ a16, const int32_t* __restrict__ b,
                             uint16_t* __restrict__ b16, int64_t cap)
{
    const int64_t n4 = cap / 4;
    const int64_t step = (int64_t)gridDim.x * blockDim.x;
    for (int64_t q = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; q < n4; q += step) {
        if (a16) {
            const int4 v = reinterpret_cast<const int4*>(a)[q];
            reinterpret_cast<uint2*>(a16)[q] = make_uint2((uint32_t)v.x | ((uint32_t)v.y << 16),
                                                          (uint32_t)v.z | ((uint32_t)v.w << 16));
        }
        if (b16) {
            const int4 v = reinterpret_cast<const int4*>(b)[q];
            reinterpret_cast<uint2*>(b16)[q] = make_uint2((uint32_t)v.x | ((uint32_t)v.y << 16),
                                                          (uint32_t)v.z | ((uint32_t)v.w << 16));
        }
    }
}

snack_status build_idx16(snack_layer* L, hipStream_t s)
{
    if (!L->fwd.idx16 && !L->tr.idx16) return SNACK_OK;
    ProfScope prof(KC_CANON, s);
    const int64_t n4 = L->cap / 4;
    hipLaunchKernelGGL(idx16_kernel, dim3(grid_for(n4 < 4096 * 256 ? n4 : 4096 * 256)), dim3(kThreads), 0, s,
                       L->fwd.idx, L->fwd.idx16, L->tr.idx, L->tr.idx16, L->cap);
    SNACK_HIP(hipGetLastError());
    return SNACK_OK;
}

snack_status canon_index_tail(snack_layer* L, hipStream_t s, bool idx16_done, bool empty_cleared)
{
    if (!idx16_done) SNACK_CHECK(build_idx16(L, s));
    L->vals_t_stale = false;
    for (int i = 0; i < kTileWidths; ++i) {
        L->fwd.split[i].valid = false;
        L->tr.split[i].valid = false;
    }
    SNACK_CHECK(build_view_partitions(L, s, empty_cleared));
    return SNACK_OK;
}

snack_status refresh_vals_t(snack_layer* L, hipStream_t s)
{
    if (L->nnz > 0) {
        ProfScope prof(KC_VALS_T_REFRESH, s);
        hipLaunchKernelGGL(refresh_vals_t_kernel, dim3(grid_for(L->nnz)), dim3(kThreads), 0, s, L->iperm, L->vals,
                           L->nnz, L->vals_t);
        SNACK_HIP(hipGetLastError());
    }
    L->vals_t_stale = false;
    return SNACK_OK;
}

snack_status invert_iperm(const snack_layer* L, int32_t* perm, hipStream_t s)
{
    if (L->nnz > 0) {
        hipLaunchKernelGGL(invert_iperm_kernel, dim3(grid_for(L->nnz)), dim3(kThreads), 0, s, L->iperm, L->nnz, perm);
        SNACK_HIP(hipGetLastError());
    }
    return SNACK_OK;
}

}  // namespace snack
