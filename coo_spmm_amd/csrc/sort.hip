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

// ---- exclusive scan: tile totals, then tiles with their prefix ----------------
// Kernel 1 reduces each tile of 4096 items (int4 loads) to its total.  Kernel
// 2 rescans each tile and adds the tile's prefix: with at most kScanDirect
// tiles the workgroup sums the totals before its tile itself (they are few
// and stay in L2); with more, the totals are first scanned in place by the
// same routine (two levels reach 2^36 items).  No atomics, no waiting.
constexpr int kScanThreads = 256;
constexpr int kScanRounds = 4;                                // int4 per thread per tile
constexpr int kScanTile = kScanThreads * 4 * kScanRounds;    // 4096 items
constexpr int64_t kScanDirect = 4096;

template <bool VEC>
__device__ inline int4 scan_load(const int32_t* __restrict__ in, int64_t e, int64_t n)
{
    int4 x;
    if (VEC && e + 3 < n) {
        x = *reinterpret_cast<const int4*>(in + e);
    } else {
        x.x = e < n ? in[e] : 0;
        x.y = e + 1 < n ? in[e + 1] : 0;
        x.z = e + 2 < n ? in[e + 2] : 0;
        x.w = e + 3 < n ? in[e + 3] : 0;
    }
    return x;
}

template <bool VEC>
__global__ void __launch_bounds__(kScanThreads) scan_tile_sums_kernel(const int32_t* __restrict__ in, int64_t n,
                                                                      int32_t* __restrict__ sums)
{
    __shared__ int32_t smem[kScanThreads / kWave];
    const int64_t base = (int64_t)blockIdx.x * kScanTile;
    int32_t s = 0;
#pragma unroll
    for (int q = 0; q < kScanRounds; ++q) {
        const int4 x = scan_load<VEC>(in, base + (int64_t)q * (kScanThreads * 4) + 4 * threadIdx.x, n);
        s += x.x + x.y + x.z + x.w;
    }
    int32_t tot;
    block_exclusive_scan<kScanThreads>(s, smem, &tot);
    if (threadIdx.x == 0) sums[blockIdx.x] = tot;
}

// Inputs of up to kScanSmallMax items in one launch: one workgroup copies them
// to LDS with coalesced loads (all in flight), each thread scans a contiguous
// run there (summed, block-scanned, then rewritten with running prefixes), and
// the result is copied back coalesced.  In and out may be the same array.
constexpr int kScanSmallThreads = 1024;
constexpr int kScanSmallPer = 16;
constexpr int64_t kScanSmallMax = (int64_t)kScanSmallPer * kScanSmallThreads;

__global__ void __launch_bounds__(kScanSmallThreads) scan_small_kernel(const int32_t* in, int32_t* out, int64_t n,
                                                                       int32_t* __restrict__ total)
{
    __shared__ int32_t buf[kScanSmallMax];
    __shared__ int32_t smem[kScanSmallThreads / kWave];
    const int tid = (int)threadIdx.x;
    const int nn = (int)n;
#pragma unroll
    for (int i = 0; i < kScanSmallPer; ++i) {
        const int e = tid + i * kScanSmallThreads;
        if (e < nn) buf[e] = in[e];
    }
    __syncthreads();
    const int per = (nn + kScanSmallThreads - 1) / kScanSmallThreads;
    const int b = tid * per;
    int32_t s = 0;
    for (int i = 0; i < per; ++i)
        if (b + i < nn) s += buf[b + i];
    int32_t tot;
    int32_t run = block_exclusive_scan<kScanSmallThreads>(s, smem, &tot);
    for (int i = 0; i < per; ++i) {
        if (b + i < nn) {
            const int32_t v = buf[b + i];
            buf[b + i] = run;
            run += v;
        }
    }
    __syncthreads();
#pragma unroll
    for (int i = 0; i < kScanSmallPer; ++i) {
        const int e = tid + i * kScanSmallThreads;
        if (e < nn) out[e] = buf[e];
    }
    if (total && tid == 0) *total = tot;
}

// direct: the tile prefix is the sum of sums[0, tile); otherwise sums holds exclusive prefixes
template <bool VEC, bool DIRECT>
__global__ void __launch_bounds__(kScanThreads) scan_tiles_kernel(const int32_t* __restrict__ in,
                                                                  int32_t* __restrict__ out, int64_t n,
                                                                  const int32_t* __restrict__ sums, int64_t ntiles,
                                                                  int32_t* __restrict__ total)
{
    __shared__ int32_t smem[kScanThreads / kWave];
    const int64_t tile = blockIdx.x;
    const int64_t base = tile * kScanTile;
    int32_t prefix;
    if constexpr (DIRECT) {
        int32_t part = 0;
        for (int64_t i = threadIdx.x; i < tile; i += kScanThreads) part += sums[i];
        int32_t tot;
        block_exclusive_scan<kScanThreads>(part, smem, &tot);
        prefix = tot;
    } else {
        prefix = sums[tile];
    }
    int4 x[kScanRounds];
    int32_t ex[kScanRounds], sub[kScanRounds];
    int32_t agg = 0;
#pragma unroll
    for (int q = 0; q < kScanRounds; ++q) {
        x[q] = scan_load<VEC>(in, base + (int64_t)q * (kScanThreads * 4) + 4 * threadIdx.x, n);
        int32_t tot;
        ex[q] = block_exclusive_scan<kScanThreads>(x[q].x + x[q].y + x[q].z + x[q].w, smem, &tot);
        sub[q] = agg;
        agg += tot;
    }
    if (total && tile == ntiles - 1 && threadIdx.x == 0) *total = prefix + agg;
#pragma unroll
    for (int q = 0; q < kScanRounds; ++q) {
        const int64_t e = base + (int64_t)q * (kScanThreads * 4) + 4 * threadIdx.x;
        int4 o;
        o.x = prefix + sub[q] + ex[q];
        o.y = o.x + x[q].x;
        o.z = o.y + x[q].y;
        o.w = o.z + x[q].z;
        if (VEC && e + 3 < n) {
            *reinterpret_cast<int4*>(out + e) = o;
        } else {
            if (e < n) out[e] = o.x;
            if (e + 1 < n) out[e + 1] = o.y;
            if (e + 2 < n) out[e + 2] = o.z;
            if (e + 3 < n) out[e + 3] = o.w;
        }
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
    size_t b = 0;
    int64_t m = n;
    do {
        const int64_t nt = (m + kScanTile - 1) / kScanTile;
        b += (((size_t)nt + 64) * 4 + 255) & ~(size_t)255;
        m = nt;
    } while (m > kScanDirect);
    return b;
}

snack_status exclusive_scan_i32(const int32_t* in, int32_t* out, int64_t n, int32_t* total_dev, void* scratch,
                                hipStream_t s)
{
    if (n <= 0) {
        if (total_dev) SNACK_HIP(hipMemsetAsync(total_dev, 0, 4, s));
        return SNACK_OK;
    }
    if (n <= kScanSmallMax) {
        hipLaunchKernelGGL(scan_small_kernel, dim3(1), dim3(kScanSmallThreads), 0, s, in, out, n, total_dev);
        SNACK_HIP(hipGetLastError());
        return SNACK_OK;
    }
    const int64_t nt = (n + kScanTile - 1) / kScanTile;
    int32_t* sums = (int32_t*)scratch;
    void* rest = (char*)scratch + ((((size_t)nt + 64) * 4 + 255) & ~(size_t)255);
    const bool vec = ((uintptr_t)in % 16 == 0) && ((uintptr_t)out % 16 == 0);
    if (vec)
        hipLaunchKernelGGL(scan_tile_sums_kernel<true>, dim3((unsigned)nt), dim3(kScanThreads), 0, s, in, n, sums);
    else
        hipLaunchKernelGGL(scan_tile_sums_kernel<false>, dim3((unsigned)nt), dim3(kScanThreads), 0, s, in, n, sums);
    SNACK_HIP(hipGetLastError());
    if (nt <= kScanDirect) {
        if (vec)
            hipLaunchKernelGGL((scan_tiles_kernel<true, true>), dim3((unsigned)nt), dim3(kScanThreads), 0, s, in, out,
                               n, sums, nt, total_dev);
        else
            hipLaunchKernelGGL((scan_tiles_kernel<false, true>), dim3((unsigned)nt), dim3(kScanThreads), 0, s, in,
                               out, n, sums, nt, total_dev);
    } else {
        SNACK_CHECK(exclusive_scan_i32(sums, sums, nt, nullptr, rest, s));
        if (vec)
            hipLaunchKernelGGL((scan_tiles_kernel<true, false>), dim3((unsigned)nt), dim3(kScanThreads), 0, s, in,
                               out, n, sums, nt, total_dev);
        else
            hipLaunchKernelGGL((scan_tiles_kernel<false, false>), dim3((unsigned)nt), dim3(kScanThreads), 0, s, in,
                               out, n, sums, nt, total_dev);
    }
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
