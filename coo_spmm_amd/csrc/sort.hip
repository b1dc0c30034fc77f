// sort.hip -- device-wide exclusive scan and stable LSD radix sort.
//
// Used by canonicalisation (sort by linear position, then a stable sort by
// column for the transposed view) and by drop/regrow (dedupe of candidate
// positions).  Stability comes from processing each tile in element order: a
// wave ranks its 64 elements per digit with ballots, waves are combined in
// order through LDS, and tiles are combined in order by the scanned
// digit-major histogram.  Integer-only, deterministic.
#include "internal.h"

#include <atomic>

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

// ---- single-pass scan (decoupled look-back) ----------------------------------
// A workgroup takes the next tile by ticket, reduces it, publishes its
// aggregate, and walks back over its predecessors' published words (64 at a
// time, one per lane of wave 0) until it meets an inclusive prefix; then it
// publishes its own inclusive prefix and writes the tile.  Each published
// word packs (call tag, status, value) so it is read and written atomically,
// and the tag lets a call ignore words left by earlier calls (no clearing).
// The words are read and written with atomic read-modify-write operations:
// those are coherent across the XCDs, where a plain load may be served by a
// stale line in the reader's own L2.
// A workgroup waits only on tickets handed out before its own, whose holders
// are already running, so the walk always ends.  The ticket counter is
// cleared by a one-thread kernel launched just before.
constexpr int kDlThreads = 256;
constexpr int kDlRounds = 4;                        // int4 per thread per tile
constexpr int kDlTile = kDlThreads * 4 * kDlRounds;  // 4096 items
constexpr uint64_t kDlAgg = 1, kDlIncl = 2;

__device__ inline uint64_t dl_word(uint32_t tag, uint64_t status, uint64_t value)
{
    return ((uint64_t)tag << 40) | (status << 38) | (value & ((1ull << 38) - 1));
}

__global__ void scan_ticket_reset_kernel(unsigned long long* __restrict__ ticket)
{
    if (threadIdx.x == 0 && blockIdx.x == 0) atomicExch(ticket, 0ull);
}

template <bool VEC>
__global__ void __launch_bounds__(kDlThreads) scan_dl_kernel(const int32_t* __restrict__ in, int32_t* __restrict__ out,
                                                             int64_t n, int32_t* __restrict__ total,
                                                             unsigned long long* __restrict__ state,
                                                             unsigned long long* __restrict__ ticket, uint32_t tag,
                                                             int64_t ntiles)
{
    __shared__ int32_t smem[kDlThreads / kWave];
    __shared__ int64_t s_tile;
    __shared__ int64_t s_prefix;
    const int lane = lane_id();
    const int w = threadIdx.x / kWave;
    if (threadIdx.x == 0) s_tile = (int64_t)atomicAdd(ticket, 1ull);
    __syncthreads();
    const int64_t tile = s_tile;
    const int64_t base = tile * kDlTile;

    int4 x[kDlRounds];
    int32_t ex[kDlRounds];
    int32_t sub[kDlRounds];
    int32_t agg = 0;
#pragma unroll
    for (int q = 0; q < kDlRounds; ++q) {
        const int64_t e = base + (int64_t)q * (kDlThreads * 4) + 4 * threadIdx.x;
        if (VEC && e + 3 < n) {
            x[q] = *reinterpret_cast<const int4*>(in + e);
        } else {
            x[q].x = e < n ? in[e] : 0;
            x[q].y = e + 1 < n ? in[e + 1] : 0;
            x[q].z = e + 2 < n ? in[e + 2] : 0;
            x[q].w = e + 3 < n ? in[e + 3] : 0;
        }
        int32_t tot;
        ex[q] = block_exclusive_scan<kDlThreads>(x[q].x + x[q].y + x[q].z + x[q].w, smem, &tot);
        sub[q] = agg;
        agg += tot;
    }

    if (w == 0) {
        int64_t prefix = 0;
        if (tile == 0) {
            if (lane == 0)
                atomicExch(&state[0], (unsigned long long)dl_word(tag, kDlIncl, (uint64_t)agg));
        } else {
            if (lane == 0)
                atomicExch(&state[tile], (unsigned long long)dl_word(tag, kDlAgg, (uint64_t)agg));
            int64_t j = tile - 1;
            for (;;) {
                const int64_t idx = j - lane;
                uint64_t st = kDlIncl, val = 0;
                if (idx >= 0) {
                    for (;;) {
                        const unsigned long long wd = atomicAdd(&state[idx], 0ull);
                        st = ((uint32_t)(wd >> 40) == tag) ? ((wd >> 38) & 3ull) : 0ull;
                        val = wd & ((1ull << 38) - 1);
                        if (st != 0) break;
                        __builtin_amdgcn_s_sleep(1);
                    }
                }
                const uint64_t incl = __ballot(st == kDlIncl);
                const int stop = incl ? __ffsll((unsigned long long)incl) - 1 : kWave - 1;
                int64_t v = lane <= stop ? (int64_t)val : 0;
#pragma unroll
                for (int d = kWave / 2; d >= 1; d >>= 1) v += __shfl_xor(v, d, kWave);
                prefix += v;
                if (incl) break;
                j -= kWave;
            }
            if (lane == 0)
                atomicExch(&state[tile], (unsigned long long)dl_word(tag, kDlIncl, (uint64_t)(prefix + agg)));
        }
        if (lane == 0) {
            s_prefix = prefix;
            if (tile == ntiles - 1 && total) *total = (int32_t)(prefix + agg);
        }
    }
    __syncthreads();
    const int32_t pre = (int32_t)s_prefix;
#pragma unroll
    for (int q = 0; q < kDlRounds; ++q) {
        const int64_t e = base + (int64_t)q * (kDlThreads * 4) + 4 * threadIdx.x;
        int4 o;
        o.x = pre + sub[q] + ex[q];
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
    const int64_t nt = (n + kDlTile - 1) / kDlTile;
    return (((size_t)nt + 1) * 8 + 255) & ~(size_t)255;
}

snack_status exclusive_scan_i32(const int32_t* in, int32_t* out, int64_t n, int32_t* total_dev, void* scratch,
                                hipStream_t s)
{
    if (n <= 0) {
        if (total_dev) SNACK_HIP(hipMemsetAsync(total_dev, 0, 4, s));
        return SNACK_OK;
    }
    // every call gets its own tag (never 0), so stale words and tickets are ignored
    static std::atomic<uint32_t> calls{0};
    uint32_t tag = (calls.fetch_add(1, std::memory_order_relaxed) + 1) & 0xFFFFFFu;
    if (tag == 0) tag = (calls.fetch_add(1, std::memory_order_relaxed) + 1) & 0xFFFFFFu;
    const int64_t nt = (n + kDlTile - 1) / kDlTile;
    unsigned long long* ticket = (unsigned long long*)scratch;
    unsigned long long* state = ticket + 1;
    const bool vec = ((uintptr_t)in % 16 == 0) && ((uintptr_t)out % 16 == 0);
    hipLaunchKernelGGL(scan_ticket_reset_kernel, dim3(1), dim3(64), 0, s, ticket);
    if (vec)
        hipLaunchKernelGGL(scan_dl_kernel<true>, dim3((unsigned)nt), dim3(kDlThreads), 0, s, in, out, n, total_dev,
                           state, ticket, tag, nt);
    else
        hipLaunchKernelGGL(scan_dl_kernel<false>, dim3((unsigned)nt), dim3(kDlThreads), 0, s, in, out, n, total_dev,
                           state, ticket, tag, nt);
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
