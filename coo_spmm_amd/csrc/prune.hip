// prune.hip -- in-place drop / regrow of connections with nnz fixed.
//
// The DST update of the "Padded-CSR" post (section 4.3: drop a fraction of the
// live entries, grow the same number elsewhere) applied in place on the COO
// triple as in the SNACK paper's Figure 1, with the SET-style rule:
//   drop   the n_drop entries of smallest |v|, in the total order of the key
//          (IEEE bits of |v|, canonical slot) -- found by an MSB-first radix
//          select over the magnitude bits plus a slot-order scan of the ties;
//   grow   n_drop positions uniform over the cells empty after the drop, value
//          +0.0: candidate t is SplitMix64 output number epoch*2^40 + t of the
//          generator seeded with the layer seed (Steele, Lea & Flood 2014),
//          mapped onto [0, M*K) by the high word of the 64x64 product; a
//          candidate is accepted if its cell is neither kept nor accepted at a
//          smaller t.  Candidates are tested in batches against an occupancy
//          bitmap; inside a batch, a stable sort by position keeps the first
//          occurrence of each cell, and a scan in t order keeps the first
//          `need` accepted -- so the result never depends on the batch size.
// The kept entries (already in canonical order) and the grown ones (sorted
// by position) are merged by a merge-path style rank search, after which the
// index structures are rebuilt.  Every step is integer work and deterministic.
#include "internal.h"

namespace snack {
namespace {

constexpr int kThreads = 256;
constexpr uint64_t kGamma = 0x9E3779B97F4A7C15ull;
constexpr int64_t kMaxBatch = 16 * 1024 * 1024;
constexpr uint64_t kMaxBitmapBits = 1ull << 34;

inline unsigned grid_for(int64_t n)
{
    int64_t g = (n + kThreads - 1) / kThreads;
    if (g < 1) g = 1;
    if (g > 65535LL * 8) g = 65535LL * 8;
    return (unsigned)g;
}

inline int bits_for(uint64_t maxval)
{
    int b = 1;
    while (b < 64 && (maxval >> b) != 0) ++b;
    return b;
}

inline size_t al(size_t b) { return (b + 255) & ~(size_t)255; }

__device__ inline uint64_t splitmix64_output(uint64_t z)
{
    z = (z ^ (z >> 30)) * 0xBF58476D1CE4E5B9ull;
    z = (z ^ (z >> 27)) * 0x94D049BB133111EBull;
    return z ^ (z >> 31);
}

__device__ inline uint32_t mag_bits(float v) { return __float_as_uint(v) & 0x7FFFFFFFu; }

// state: [0] prefix, [1] rank still to find among keys matching the prefix
__global__ void sel_hist_kernel(const float* __restrict__ vals, int64_t n, const uint32_t* __restrict__ state,
                                int shift, uint32_t* __restrict__ hist)
{
    __shared__ uint32_t h[256];
    h[threadIdx.x] = 0;
    __syncthreads();
    const uint32_t prefix = state[0];
    const uint32_t hi_mask = (shift >= 24) ? 0u : (0xFFFFFFFFu << (shift + 8));
    for (int64_t k = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; k < n; k += (int64_t)gridDim.x * blockDim.x) {
        const uint32_t key = mag_bits(vals[k]);
        if ((key & hi_mask) == (prefix & hi_mask)) atomicAdd(&h[(key >> shift) & 255u], 1u);
    }
    __syncthreads();
    if (h[threadIdx.x]) atomicAdd(&hist[threadIdx.x], h[threadIdx.x]);
}

__global__ void sel_pick_kernel(uint32_t* __restrict__ hist, uint32_t* __restrict__ state, int shift)
{
    if (threadIdx.x != 0 || blockIdx.x != 0) return;
    uint32_t r = state[1];
    uint32_t d = 0;
    for (; d < 256; ++d) {
        if (r < hist[d]) break;
        r -= hist[d];
    }
    state[0] |= d << shift;
    state[1] = r;
    for (int i = 0; i < 256; ++i) hist[i] = 0;
}

__global__ void eq_flags_kernel(const float* __restrict__ vals, int64_t n, const uint32_t* __restrict__ state,
                                int32_t* __restrict__ eq)
{
    const uint32_t T = state[0];
    for (int64_t k = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; k < n; k += (int64_t)gridDim.x * blockDim.x)
        eq[k] = mag_bits(vals[k]) == T ? 1 : 0;
}

// keep[k] = 0 for the dropped entries: key < T, or key == T among the first (rank+1) ties in slot order
__global__ void keep_flags_kernel(const float* __restrict__ vals, int64_t n, const uint32_t* __restrict__ state,
                                  const int32_t* __restrict__ eqrank, int32_t* __restrict__ keep)
{
    const uint32_t T = state[0];
    const uint32_t ties = state[1] + 1;
    for (int64_t k = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; k < n; k += (int64_t)gridDim.x * blockDim.x) {
        const uint32_t key = mag_bits(vals[k]);
        const bool drop = key < T || (key == T && (uint32_t)eqrank[k] < ties);
        keep[k] = drop ? 0 : 1;
    }
}

__global__ void fill_u32_kernel(uint32_t* __restrict__ p, int64_t n, uint32_t v)
{
    for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < n; i += (int64_t)gridDim.x * blockDim.x)
        p[i] = v;
}

__global__ void compact_kept_kernel(const int32_t* __restrict__ rows, const int32_t* __restrict__ cols,
                                    const float* __restrict__ vals, int64_t n, int32_t K,
                                    const int32_t* __restrict__ keep, const int32_t* __restrict__ kidx,
                                    uint64_t* __restrict__ kpos, float* __restrict__ kval,
                                    uint32_t* __restrict__ bitmap)
{
    for (int64_t k = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; k < n; k += (int64_t)gridDim.x * blockDim.x) {
        if (!keep[k]) continue;
        const uint64_t p = (uint64_t)rows[k] * (uint64_t)K + (uint64_t)cols[k];
        const int32_t i = kidx[k];
        kpos[i] = p;
        kval[i] = vals[k];
        atomicOr(&bitmap[p >> 5], 1u << (p & 31));
    }
}

// candidate i of this batch is stream element t0 + i; occupied cells get the sentinel key N
__global__ void gen_candidates_kernel(uint64_t seed, uint64_t epoch, uint64_t t0, int64_t T, uint64_t N,
                                      const uint32_t* __restrict__ bitmap, uint64_t* __restrict__ cpos,
                                      uint32_t* __restrict__ cidx)
{
    for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < T; i += (int64_t)gridDim.x * blockDim.x) {
        const uint64_t t = t0 + (uint64_t)i;
        const uint64_t x = seed + ((epoch << 40) + t + 1ull) * kGamma;
        const uint64_t pos = __umul64hi(splitmix64_output(x), N);
        const bool occupied = (bitmap[pos >> 5] >> (pos & 31)) & 1u;
        cpos[i] = occupied ? N : pos;
        cidx[i] = (uint32_t)i;
    }
}

// after the stable sort by position: first occurrence of each free cell marks its candidate index
__global__ void first_occurrence_kernel(const uint64_t* __restrict__ spos, const uint32_t* __restrict__ sidx,
                                        int64_t T, uint64_t N, int32_t* __restrict__ accepted)
{
    for (int64_t j = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; j < T; j += (int64_t)gridDim.x * blockDim.x) {
        const uint64_t p = spos[j];
        const bool first = p < N && (j == 0 || spos[j - 1] != p);
        accepted[sidx[j]] = first ? 1 : 0;
    }
}

// in position order: keep the accepted candidates whose rank in t order is below `need`
__global__ void final_flags_kernel(const uint64_t* __restrict__ spos, const uint32_t* __restrict__ sidx, int64_t T,
                                   uint64_t N, const int32_t* __restrict__ accepted, const int32_t* __restrict__ trank,
                                   int64_t need, int32_t* __restrict__ fin)
{
    for (int64_t j = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; j < T; j += (int64_t)gridDim.x * blockDim.x) {
        const uint64_t p = spos[j];
        const uint32_t i = sidx[j];
        fin[j] = (p < N && accepted[i] && (int64_t)trank[i] < need) ? 1 : 0;
    }
}

__global__ void emit_grown_kernel(const uint64_t* __restrict__ spos, int64_t T, const int32_t* __restrict__ fin,
                                  const int32_t* __restrict__ fidx, uint64_t* __restrict__ grown, int64_t gbase,
                                  uint32_t* __restrict__ bitmap)
{
    for (int64_t j = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; j < T; j += (int64_t)gridDim.x * blockDim.x) {
        if (!fin[j]) continue;
        const uint64_t p = spos[j];
        grown[gbase + fidx[j]] = p;
        atomicOr(&bitmap[p >> 5], 1u << (p & 31));
    }
}

__device__ inline int64_t lower_bound_u64(const uint64_t* __restrict__ a, int64_t n, uint64_t x)
{
    int64_t lo = 0, hi = n;
    while (lo < hi) {
        const int64_t mid = lo + ((hi - lo) >> 1);
        if (a[mid] < x) lo = mid + 1;
        else hi = mid;
    }
    return lo;
}

__global__ void merge_kept_kernel(const uint64_t* __restrict__ kpos, const float* __restrict__ kval, int64_t nk,
                                  const uint64_t* __restrict__ grown, int64_t ng, int32_t K, int32_t* __restrict__ rows,
                                  int32_t* __restrict__ cols, float* __restrict__ vals)
{
    for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < nk; i += (int64_t)gridDim.x * blockDim.x) {
        const uint64_t p = kpos[i];
        const int64_t o = i + lower_bound_u64(grown, ng, p);
        rows[o] = (int32_t)(p / (uint64_t)K);
        cols[o] = (int32_t)(p % (uint64_t)K);
        vals[o] = kval[i];
    }
}

__global__ void merge_grown_kernel(const uint64_t* __restrict__ kpos, int64_t nk, const uint64_t* __restrict__ grown,
                                   int64_t ng, int32_t K, int32_t* __restrict__ rows, int32_t* __restrict__ cols,
                                   float* __restrict__ vals)
{
    for (int64_t j = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; j < ng; j += (int64_t)gridDim.x * blockDim.x) {
        const uint64_t p = grown[j];
        const int64_t o = j + lower_bound_u64(kpos, nk, p);
        rows[o] = (int32_t)(p / (uint64_t)K);
        cols[o] = (int32_t)(p % (uint64_t)K);
        vals[o] = 0.0f;
    }
}

struct PruneScratch {
    uint32_t* hist;     // [256]
    uint32_t* state;    // [16]
    int32_t* count;     // [4]
    int32_t* a;         // [nnz] flags / eq
    int32_t* b;         // [nnz] scan result
    int32_t* keep;      // [nnz]
    uint64_t* kpos;     // [nnz]
    float* kval;        // [nnz]
    uint64_t* grown;    // [nnz]
    uint32_t* bitmap;   // [(N+31)/32]
    uint64_t* cpos;     // [Tm]
    uint32_t* cidx;     // [Tm]
    int32_t* acc;       // [Tm]
    int32_t* trank;     // [Tm]
    int32_t* fin;       // [Tm]
    int32_t* fidx;      // [Tm]
    void* sort;         // sort + scan scratch
    int64_t tmax;
};

int64_t batch_cap(const snack_layer* L)
{
    int64_t t = L->nnz + 4096;
    if (t < 65536) t = 65536;
    if (t > kMaxBatch) t = kMaxBatch;
    return t;
}

size_t layout(const snack_layer* L, PruneScratch* ps)
{
    const int64_t n = L->nnz > 0 ? L->nnz : 1;
    const uint64_t N = (uint64_t)L->M * (uint64_t)L->K;
    const int64_t words = (int64_t)((N + 31) / 32);
    const int64_t tm = batch_cap(L);
    const int kb = bits_for(N);
    size_t sortb = radix_sort_scratch_bytes(tm > n ? tm : n, kb > 32 ? 64 : 33);
    size_t scanb = scan_scratch_bytes(tm > n ? tm : n);
    size_t sub = sortb > scanb ? sortb : scanb;
    size_t off = 0;
    auto take = [&](size_t bytes) {
        size_t o = off;
        off += al(bytes);
        return o;
    };
    size_t o_hist = take(256 * 4), o_state = take(16 * 4), o_count = take(16);
    size_t o_a = take((size_t)n * 4), o_b = take((size_t)n * 4), o_keep = take((size_t)n * 4);
    size_t o_kpos = take((size_t)n * 8), o_kval = take((size_t)n * 4), o_grown = take((size_t)n * 8);
    size_t o_bitmap = take((size_t)words * 4);
    size_t o_cpos = take((size_t)tm * 8), o_cidx = take((size_t)tm * 4), o_acc = take((size_t)tm * 4);
    size_t o_trank = take((size_t)tm * 4), o_fin = take((size_t)tm * 4), o_fidx = take((size_t)tm * 4);
    size_t o_sort = take(sub);
    if (ps) {
        char* base = (char*)L->scratch;
        ps->hist = (uint32_t*)(base + o_hist);
        ps->state = (uint32_t*)(base + o_state);
        ps->count = (int32_t*)(base + o_count);
        ps->a = (int32_t*)(base + o_a);
        ps->b = (int32_t*)(base + o_b);
        ps->keep = (int32_t*)(base + o_keep);
        ps->kpos = (uint64_t*)(base + o_kpos);
        ps->kval = (float*)(base + o_kval);
        ps->grown = (uint64_t*)(base + o_grown);
        ps->bitmap = (uint32_t*)(base + o_bitmap);
        ps->cpos = (uint64_t*)(base + o_cpos);
        ps->cidx = (uint32_t*)(base + o_cidx);
        ps->acc = (int32_t*)(base + o_acc);
        ps->trank = (int32_t*)(base + o_trank);
        ps->fin = (int32_t*)(base + o_fin);
        ps->fidx = (int32_t*)(base + o_fidx);
        ps->sort = base + o_sort;
        ps->tmax = tm;
    }
    return off + 256;
}

}  // namespace

size_t prune_scratch_bytes(const snack_layer* L)
{
    const uint64_t N = (uint64_t)L->M * (uint64_t)L->K;
    if (N > kMaxBitmapBits) return 0;
    return layout(L, nullptr);
}

snack_status prune_regrow(snack_layer* L, int64_t n_drop, hipStream_t s)
{
    const int64_t nnz = L->nnz;
    const uint64_t N = (uint64_t)L->M * (uint64_t)L->K;
    if (n_drop == 0) {
        L->epoch += 1;
        return SNACK_OK;
    }
    if (N > kMaxBitmapBits || L->scratch_bytes < layout(L, nullptr)) return SNACK_ERR_UNSUPPORTED;
    ProfScope prof(KC_PRUNE, s);
    PruneScratch ps;
    layout(L, &ps);
    const int64_t kept = nnz - n_drop;

    // ---- drop: the n_drop-th smallest magnitude key T and its tie rank ----
    {
        uint32_t init[2] = {0u, (uint32_t)(n_drop - 1)};
        SNACK_HIP(hipMemcpyAsync(ps.state, init, sizeof init, hipMemcpyHostToDevice, s));
        hipLaunchKernelGGL(fill_u32_kernel, dim3(1), dim3(kThreads), 0, s, ps.hist, (int64_t)256, 0u);
        for (int shift = 24; shift >= 0; shift -= 8) {
            hipLaunchKernelGGL(sel_hist_kernel, dim3(grid_for(nnz) > 2048 ? 2048 : grid_for(nnz)), dim3(kThreads), 0,
                               s, L->vals, nnz, ps.state, shift, ps.hist);
            hipLaunchKernelGGL(sel_pick_kernel, dim3(1), dim3(64), 0, s, ps.hist, ps.state, shift);
        }
        SNACK_HIP(hipGetLastError());
        hipLaunchKernelGGL(eq_flags_kernel, dim3(grid_for(nnz)), dim3(kThreads), 0, s, L->vals, nnz, ps.state, ps.a);
        SNACK_CHECK(exclusive_scan_i32(ps.a, ps.b, nnz, nullptr, ps.sort, s));
        hipLaunchKernelGGL(keep_flags_kernel, dim3(grid_for(nnz)), dim3(kThreads), 0, s, L->vals, nnz, ps.state, ps.b,
                           ps.keep);
        SNACK_CHECK(exclusive_scan_i32(ps.keep, ps.b, nnz, nullptr, ps.sort, s));
        const int64_t words = (int64_t)((N + 31) / 32);
        hipLaunchKernelGGL(fill_u32_kernel, dim3(grid_for(words)), dim3(kThreads), 0, s, ps.bitmap, words, 0u);
        hipLaunchKernelGGL(compact_kept_kernel, dim3(grid_for(nnz)), dim3(kThreads), 0, s, L->rows, L->cols, L->vals,
                           nnz, L->K, ps.keep, ps.b, ps.kpos, ps.kval, ps.bitmap);
        SNACK_HIP(hipGetLastError());
    }

    // ---- grow: walk the candidate stream in batches ----
    int64_t need = n_drop;
    int64_t got = 0;
    uint64_t t0 = 0;
    int batches = 0;
    const int kb = bits_for(N);   // the sentinel N needs bits_for(N) bits
    while (need > 0) {
        const double p_empty = (double)(N - (uint64_t)kept - (uint64_t)got) / (double)N;
        double want = (double)need / (p_empty > 1e-9 ? p_empty : 1e-9) * 1.03 + 4096.0;
        int64_t T = want > (double)ps.tmax ? ps.tmax : (int64_t)want;
        if (T < 1) T = 1;
        hipLaunchKernelGGL(gen_candidates_kernel, dim3(grid_for(T)), dim3(kThreads), 0, s, L->seed, L->epoch, t0, T, N,
                           ps.bitmap, ps.cpos, ps.cidx);
        SNACK_HIP(hipGetLastError());
        SNACK_CHECK(radix_sort_u64(ps.cpos, ps.cidx, T, kb, ps.sort, s));
        hipLaunchKernelGGL(first_occurrence_kernel, dim3(grid_for(T)), dim3(kThreads), 0, s, ps.cpos, ps.cidx, T, N,
                           ps.acc);
        SNACK_CHECK(exclusive_scan_i32(ps.acc, ps.trank, T, nullptr, ps.sort, s));
        hipLaunchKernelGGL(final_flags_kernel, dim3(grid_for(T)), dim3(kThreads), 0, s, ps.cpos, ps.cidx, T, N, ps.acc,
                           ps.trank, need, ps.fin);
        SNACK_CHECK(exclusive_scan_i32(ps.fin, ps.fidx, T, ps.count, ps.sort, s));
        hipLaunchKernelGGL(emit_grown_kernel, dim3(grid_for(T)), dim3(kThreads), 0, s, ps.cpos, T, ps.fin, ps.fidx,
                           ps.grown, got, ps.bitmap);
        SNACK_HIP(hipGetLastError());
        int32_t accepted = 0;
        SNACK_HIP(hipMemcpyAsync(&accepted, ps.count, 4, hipMemcpyDeviceToHost, s));
        SNACK_HIP(hipStreamSynchronize(s));
        got += accepted;
        need -= accepted;
        t0 += (uint64_t)T;
        if (++batches > 100000) return SNACK_ERR_UNSUPPORTED;
    }
    if (batches > 1) {
        // grown positions of different batches are each sorted; sort the union by position
        uint32_t* payload = (uint32_t*)ps.a;   // any payload of nnz words; only the keys matter
        SNACK_CHECK(radix_sort_u64(ps.grown, payload, n_drop, bits_for(N - 1), ps.sort, s));
    }

    // ---- merge kept and grown into the canonical arrays ----
    hipLaunchKernelGGL(merge_kept_kernel, dim3(grid_for(kept)), dim3(kThreads), 0, s, ps.kpos, ps.kval, kept,
                       ps.grown, n_drop, L->K, L->rows, L->cols, L->vals);
    hipLaunchKernelGGL(merge_grown_kernel, dim3(grid_for(n_drop)), dim3(kThreads), 0, s, ps.kpos, kept, ps.grown,
                       n_drop, L->K, L->rows, L->cols, L->vals);
    SNACK_HIP(hipGetLastError());
    SNACK_CHECK(canon_build_index(L, s));
    L->epoch += 1;
    return SNACK_OK;
}

}  // namespace snack
