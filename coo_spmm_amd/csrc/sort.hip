// sort.hip -- device-wide exclusive scan and stable LSD radix sort.
//
// Used by canonicalisation (sort by linear position, then a stable sort by
// column for the transposed view) and by drop/regrow (dedupe of candidate
// positions).  Stability comes from processing each tile in element order: a
// wave ranks its 64 elements per digit with ballots, waves are combined in
// order through LDS, and tiles are combined in order by the scanned
// digit-major histogram.  Integer-only, deterministic.
#include "internal.h"

namespace snack {
namespace {

constexpr int kScanThreads = 256;
constexpr int kScanItems = 8;
constexpr int kScanTile = kScanThreads * kScanItems;

constexpr int kSortThreads = 256;
constexpr int kSortItems = 8;
constexpr int kSortTile = kSortThreads * kSortItems;
constexpr int kDigitBits = 8;
constexpr int kBins = 1 << kDigitBits;

__device__ inline int lane_id() { return threadIdx.x & (kWave - 1); }

// Inclusive scan across one wavefront.
__device__ inline int32_t wave_inclusive_scan(int32_t v)
{
    const int lane = lane_id();
#pragma unroll
    for (int d = 1; d < kWave; d <<= 1) {
        int32_t o = __shfl_up(v, d, kWave);
        if (lane >= d) v += o;
    }
    return v;
}

// Exclusive scan of one value per thread across the block; returns the
// exclusive prefix and writes the block total to *total.
template <int THREADS>
__device__ inline int32_t block_exclusive_scan(int32_t v, int32_t* smem /*[THREADS/64]*/, int32_t* total)
{
    const int lane = lane_id();
    const int w = threadIdx.x / kWave;
    int32_t inc = wave_inclusive_scan(v);
    if (lane == kWave - 1) smem[w] = inc;
    __syncthreads();
    int32_t wave_base = 0, sum = 0;
#pragma unroll
    for (int i = 0; i < THREADS / kWave; ++i) {
        int32_t s = smem[i];
        if (i < w) wave_base += s;
        sum += s;
    }
    __syncthreads();
    *total = sum;
    return wave_base + inc - v;
}

__global__ void __launch_bounds__(kScanThreads) scan_reduce_kernel(const int32_t* __restrict__ in, int64_t n,
                                                                   int32_t* __restrict__ partial)
{
    __shared__ int32_t smem[kScanThreads / kWave];
    const int64_t base = (int64_t)blockIdx.x * kScanTile;
    int32_t s = 0;
#pragma unroll
    for (int i = 0; i < kScanItems; ++i) {
        int64_t e = base + (int64_t)i * kScanThreads + threadIdx.x;
        if (e < n) s += in[e];
    }
    int32_t tot;
    block_exclusive_scan<kScanThreads>(s, smem, &tot);
    if (threadIdx.x == 0) partial[blockIdx.x] = tot;
}

// Single block: exclusive scan of the partials in place, total to *total.
__global__ void __launch_bounds__(kScanThreads) scan_partials_kernel(int32_t* __restrict__ partial, int64_t np,
                                                                     int32_t* __restrict__ total)
{
    __shared__ int32_t smem[kScanThreads / kWave];
    int32_t carry = 0;
    for (int64_t base = 0; base < np; base += kScanThreads) {
        int64_t e = base + threadIdx.x;
        int32_t v = e < np ? partial[e] : 0;
        int32_t tot;
        int32_t ex = block_exclusive_scan<kScanThreads>(v, smem, &tot);
        if (e < np) partial[e] = carry + ex;
        carry += tot;
    }
    if (threadIdx.x == 0 && total) *total = carry;
}

__global__ void __launch_bounds__(kScanThreads) scan_apply_kernel(const int32_t* __restrict__ in, int64_t n,
                                                                  const int32_t* __restrict__ partial,
                                                                  int32_t* __restrict__ out)
{
    __shared__ int32_t smem[kScanThreads / kWave];
    const int64_t base = (int64_t)blockIdx.x * kScanTile + (int64_t)threadIdx.x * kScanItems;
    int32_t v[kScanItems];
    int32_t s = 0;
#pragma unroll
    for (int i = 0; i < kScanItems; ++i) {
        int64_t e = base + i;
        v[i] = e < n ? in[e] : 0;
        s += v[i];
    }
    int32_t tot;
    int32_t ex = block_exclusive_scan<kScanThreads>(s, smem, &tot);
    int32_t run = partial[blockIdx.x] + ex;
#pragma unroll
    for (int i = 0; i < kScanItems; ++i) {
        int64_t e = base + i;
        if (e < n) out[e] = run;
        run += v[i];
    }
}

// ---- radix sort ------------------------------------------------------------

template <typename KeyT>
__global__ void __launch_bounds__(kSortThreads) rs_hist_kernel(const KeyT* __restrict__ keys, int64_t n, int shift,
                                                               int32_t* __restrict__ hist, int64_t nblocks)
{
    __shared__ int32_t h[kBins];
    for (int i = threadIdx.x; i < kBins; i += kSortThreads) h[i] = 0;
    __syncthreads();
    const int64_t base = (int64_t)blockIdx.x * kSortTile;
#pragma unroll
    for (int i = 0; i < kSortItems; ++i) {
        int64_t e = base + (int64_t)i * kSortThreads + threadIdx.x;
        if (e < n) {
            int d = (int)((keys[e] >> shift) & (kBins - 1));
            atomicAdd(&h[d], 1);
        }
    }
    __syncthreads();
    for (int i = threadIdx.x; i < kBins; i += kSortThreads) hist[(int64_t)i * nblocks + blockIdx.x] = h[i];
}

template <typename KeyT>
__global__ void __launch_bounds__(kSortThreads) rs_scatter_kernel(const KeyT* __restrict__ kin,
                                                                  const uint32_t* __restrict__ vin,
                                                                  KeyT* __restrict__ kout, uint32_t* __restrict__ vout,
                                                                  int64_t n, int shift,
                                                                  const int32_t* __restrict__ offs, int64_t nblocks)
{
    constexpr int W = kSortThreads / kWave;
    __shared__ int32_t gofs[kBins];
    __shared__ int32_t wcnt[W][kBins];
    for (int i = threadIdx.x; i < kBins; i += kSortThreads) gofs[i] = offs[(int64_t)i * nblocks + blockIdx.x];
    const int lane = lane_id();
    const int w = threadIdx.x / kWave;
    const uint64_t lt_mask = (lane == 0) ? 0ull : (~0ull >> (kWave - lane));
    const int64_t base = (int64_t)blockIdx.x * kSortTile;
    for (int r = 0; r < kSortItems; ++r) {
        for (int i = threadIdx.x; i < W * kBins; i += kSortThreads) (&wcnt[0][0])[i] = 0;
        __syncthreads();
        const int64_t e = base + (int64_t)r * kSortThreads + threadIdx.x;
        const bool valid = e < n;
        KeyT key = valid ? kin[e] : KeyT(0);
        uint32_t val = valid ? vin[e] : 0u;
        const int d = (int)((key >> shift) & (kBins - 1));
        uint64_t match = __ballot(valid);
#pragma unroll
        for (int b = 0; b < kDigitBits; ++b) {
            const bool bit = (d >> b) & 1;
            const uint64_t m = __ballot(bit);
            match &= bit ? m : ~m;
        }
        const int rank = __popcll(match & lt_mask);
        if (valid && rank == 0) wcnt[w][d] = __popcll(match);
        __syncthreads();
        // per digit: turn the wave counts into exclusive bases, advance gofs
        for (int dg = threadIdx.x; dg < kBins; dg += kSortThreads) {
            int32_t s = gofs[dg];
#pragma unroll
            for (int q = 0; q < W; ++q) {
                int32_t c = wcnt[q][dg];
                wcnt[q][dg] = s;
                s += c;
            }
            gofs[dg] = s;
        }
        __syncthreads();
        if (valid) {
            const int32_t pos = wcnt[w][d] + rank;
            kout[pos] = key;
            vout[pos] = val;
        }
        __syncthreads();
    }
}

template <typename KeyT>
snack_status radix_sort_impl(KeyT* keys, uint32_t* vals, int64_t n, int key_bits, void* scratch, hipStream_t s)
{
    if (n <= 1) return SNACK_OK;
    const int64_t nblocks = (n + kSortTile - 1) / kSortTile;
    char* p = (char*)scratch;
    KeyT* k2 = (KeyT*)p;
    p += ((size_t)n * sizeof(KeyT) + 255) & ~(size_t)255;
    uint32_t* v2 = (uint32_t*)p;
    p += ((size_t)n * 4 + 255) & ~(size_t)255;
    int32_t* hist = (int32_t*)p;
    p += ((size_t)nblocks * kBins * 4 + 255) & ~(size_t)255;
    void* scan_scr = p;
    KeyT* ka = keys;
    uint32_t* va = vals;
    KeyT* kb = k2;
    uint32_t* vb = v2;
    const int passes = (key_bits + kDigitBits - 1) / kDigitBits;
    ProfScope prof(KC_SORT, s);
    for (int pass = 0; pass < passes; ++pass) {
        const int shift = pass * kDigitBits;
        hipLaunchKernelGGL(rs_hist_kernel<KeyT>, dim3((unsigned)nblocks), dim3(kSortThreads), 0, s, ka, n, shift,
                           hist, nblocks);
        SNACK_HIP(hipGetLastError());
        SNACK_CHECK(exclusive_scan_i32(hist, hist, nblocks * kBins, nullptr, scan_scr, s));
        hipLaunchKernelGGL(rs_scatter_kernel<KeyT>, dim3((unsigned)nblocks), dim3(kSortThreads), 0, s, ka, va, kb,
                           vb, n, shift, hist, nblocks);
        SNACK_HIP(hipGetLastError());
        KeyT* tk = ka; ka = kb; kb = tk;
        uint32_t* tv = va; va = vb; vb = tv;
    }
    if (ka != keys) {
        SNACK_HIP(hipMemcpyAsync(keys, ka, (size_t)n * sizeof(KeyT), hipMemcpyDeviceToDevice, s));
        SNACK_HIP(hipMemcpyAsync(vals, va, (size_t)n * 4, hipMemcpyDeviceToDevice, s));
    }
    return SNACK_OK;
}

}  // namespace

size_t scan_scratch_bytes(int64_t n)
{
    int64_t nb = (n + kScanTile - 1) / kScanTile;
    return ((size_t)(nb + 1) * 4 + 255) & ~(size_t)255;
}

snack_status exclusive_scan_i32(const int32_t* in, int32_t* out, int64_t n, int32_t* total_dev, void* scratch,
                                hipStream_t s)
{
    if (n <= 0) {
        if (total_dev) SNACK_HIP(hipMemsetAsync(total_dev, 0, 4, s));
        return SNACK_OK;
    }
    const int64_t nb = (n + kScanTile - 1) / kScanTile;
    int32_t* partial = (int32_t*)scratch;
    hipLaunchKernelGGL(scan_reduce_kernel, dim3((unsigned)nb), dim3(kScanThreads), 0, s, in, n, partial);
    SNACK_HIP(hipGetLastError());
    hipLaunchKernelGGL(scan_partials_kernel, dim3(1), dim3(kScanThreads), 0, s, partial, nb, total_dev);
    SNACK_HIP(hipGetLastError());
    hipLaunchKernelGGL(scan_apply_kernel, dim3((unsigned)nb), dim3(kScanThreads), 0, s, in, n, partial, out);
    SNACK_HIP(hipGetLastError());
    return SNACK_OK;
}

size_t radix_sort_scratch_bytes(int64_t n, int key_bits)
{
    const size_t kw = key_bits > 32 ? 8 : 4;
    const int64_t nblocks = (n + kSortTile - 1) / kSortTile;
    size_t b = 0;
    b += ((size_t)n * kw + 255) & ~(size_t)255;
    b += ((size_t)n * 4 + 255) & ~(size_t)255;
    b += ((size_t)nblocks * kBins * 4 + 255) & ~(size_t)255;
    b += scan_scratch_bytes(nblocks * kBins);
    return b + 256;
}

snack_status radix_sort_u32(uint32_t* keys, uint32_t* vals, int64_t n, int key_bits, void* scratch, hipStream_t s)
{
    return radix_sort_impl<uint32_t>(keys, vals, n, key_bits, scratch, s);
}

snack_status radix_sort_u64(uint64_t* keys, uint32_t* vals, int64_t n, int key_bits, void* scratch, hipStream_t s)
{
    return radix_sort_impl<uint64_t>(keys, vals, n, key_bits, scratch, s);
}

}  // namespace snack
