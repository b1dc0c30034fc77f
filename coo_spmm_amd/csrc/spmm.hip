// spmm.hip -- segmented SpMM over a sorted view of the COO triple, and the
// sampled dense-dense product for dW.
//
// Forward (SNACK paper, Figure 1; "Padded-CSR" section 6.1) and the input
// gradient ("Padded-CSR" section 7.1, run over the transposed view of section
// 7.2) are one kernel: out[b, key] = sum of v * feat[idx, b] over the entries
// of each key, for a view sorted by key.
//
// Mapping (one wavefront per key-aligned chunk):
//  * a wave is G = 64/BT lane groups of BT lanes; each lane owns NB
//    consecutive batch columns, so a group covers a batch tile of BT*NB
//    columns and every (key, idx, value) load is shared by the whole tile;
//  * per wave step, group g takes a run of U consecutive entries, loaded as
//    16-byte vectors, so the G runs of a step stream one contiguous span of
//    the index and value arrays;
//  * the activations are feature-major (feat[idx * bp + b]) so the NB values
//    a lane gathers per entry are one vector load;
//  * a lane sums its run sequentially per key, then the groups combine run
//    tails with a segmented Hillis-Steele scan over wavefront shuffles; a key
//    still open at the end of a step is carried into the next step.  Every
//    output row is written exactly once, by plain stores: no atomics, so the
//    result is bit-reproducible.
// Chunks never split a key, so no cross-wave fix-up exists.  Workgroups are
// remapped so that each XCD streams one contiguous range of chunks.
#include "internal.h"

#include <limits.h>

namespace snack {
namespace {

constexpr int kBlock = 256;
constexpr int kWavesPerBlock = kBlock / kWave;
constexpr int kXcd = 8;

template <int NB>
__device__ inline void load_nb(const float* __restrict__ p, float (&x)[NB])
{
    if constexpr (NB == 4) {
        const float4 v = *reinterpret_cast<const float4*>(p);
        x[0] = v.x; x[1] = v.y; x[2] = v.z; x[3] = v.w;
    } else if constexpr (NB == 2) {
        const float2 v = *reinterpret_cast<const float2*>(p);
        x[0] = v.x; x[1] = v.y;
    } else {
        x[0] = *p;
    }
}

template <int BT, int NB, int U>
__global__ void __launch_bounds__(kBlock) spmm_seg_kernel(
    const int32_t* __restrict__ keys, const int32_t* __restrict__ idx, const float* __restrict__ vals,
    const int32_t* __restrict__ ptr, const int32_t* __restrict__ chunk_key, int32_t nchunks,
    const float* __restrict__ feat, int bp, int B, int32_t nkeys, float* __restrict__ out, int per_xcd,
    int nblocks)
{
    static_assert(U % 4 == 0, "runs are loaded as 16-byte vectors");
    constexpr int G = kWave / BT;
    constexpr int STEP = G * U;
    const int lane = threadIdx.x & (kWave - 1);
    const int g = lane / BT;
    const int bl = lane - g * BT;

    const int bid = (int)blockIdx.x;
    const int vb = (bid % kXcd) * per_xcd + bid / kXcd;
    if (vb >= nblocks) return;
    const int c = vb * kWavesPerBlock + (int)(threadIdx.x / kWave);
    if (c >= nchunks) return;
    const int32_t r0 = chunk_key[c];
    const int32_t r1 = chunk_key[c + 1];
    if (r0 >= r1) return;

    const int tile0 = (int)blockIdx.y * (BT * NB);
    const int bcol = tile0 + bl * NB;
    const float* __restrict__ fb = feat + bcol;

    auto write_row = [&](int32_t key, const float (&a)[NB]) {
        if (key >= r0 && key < r1) {
#pragma unroll
            for (int n = 0; n < NB; ++n) {
                const int b = bcol + n;
                if (b < B) out[(int64_t)b * nkeys + key] = a[n];
            }
        }
    };

    // keys of this chunk with no entry produce zeros
    for (int32_t r = r0 + lane; r < r1; r += kWave) {
        if (ptr[r] == ptr[r + 1]) {
            for (int q = 0; q < BT * NB; ++q) {
                const int b = tile0 + q;
                if (b < B) out[(int64_t)b * nkeys + r] = 0.0f;
            }
        }
    }

    const int64_t s = ptr[r0];
    const int64_t e = ptr[r1];
    int32_t carry_key = -1;
    float carry[NB];
#pragma unroll
    for (int n = 0; n < NB; ++n) carry[n] = 0.0f;

    for (int64_t base = s & ~(int64_t)3; base < e; base += STEP) {
        const int64_t my = base + (int64_t)g * U;
        int32_t key[U], ix[U];
        float v[U];
#pragma unroll
        for (int q = 0; q < U / 4; ++q) {
            const int4 kk = *reinterpret_cast<const int4*>(keys + my + 4 * q);
            const int4 ii = *reinterpret_cast<const int4*>(idx + my + 4 * q);
            const float4 vv = *reinterpret_cast<const float4*>(vals + my + 4 * q);
            key[4 * q + 0] = kk.x; key[4 * q + 1] = kk.y; key[4 * q + 2] = kk.z; key[4 * q + 3] = kk.w;
            ix[4 * q + 0] = ii.x; ix[4 * q + 1] = ii.y; ix[4 * q + 2] = ii.z; ix[4 * q + 3] = ii.w;
            v[4 * q + 0] = vv.x; v[4 * q + 1] = vv.y; v[4 * q + 2] = vv.z; v[4 * q + 3] = vv.w;
        }
#pragma unroll
        for (int u = 0; u < U; ++u) {
            const int64_t k = my + u;
            if (k < s || k >= e) {
                key[u] = (k < s) ? -1 : INT_MAX;
                ix[u] = 0;
                v[u] = 0.0f;
            }
        }
        float x[U][NB];
#pragma unroll
        for (int u = 0; u < U; ++u) load_nb<NB>(fb + (int64_t)ix[u] * bp, x[u]);

        // sequential per-key sums along the run
        float head[NB], acc[NB];
        bool multi = false;
#pragma unroll
        for (int n = 0; n < NB; ++n) {
            acc[n] = v[0] * x[0][n];
            head[n] = 0.0f;
        }
#pragma unroll
        for (int u = 1; u < U; ++u) {
            if (key[u] != key[u - 1]) {
                if (multi) {
                    write_row(key[u - 1], acc);   // a key wholly inside this run
                } else {
#pragma unroll
                    for (int n = 0; n < NB; ++n) head[n] = acc[n];
                    multi = true;
                }
#pragma unroll
                for (int n = 0; n < NB; ++n) acc[n] = v[u] * x[u][n];
            } else {
#pragma unroll
                for (int n = 0; n < NB; ++n) acc[n] = fmaf(v[u], x[u][n], acc[n]);
            }
        }
        const int32_t head_key = key[0];
        const int32_t tail_key = key[U - 1];

        // the open key carried from the previous step is complete unless this step continues it
        const int32_t first_key = __shfl(head_key, 0, kWave);
        if (g == 0 && carry_key != first_key) write_row(carry_key, carry);

        int32_t ptail = __shfl_up(tail_key, BT, kWave);
        if (g == 0) ptail = carry_key;
        int f = (multi || ptail != tail_key) ? 1 : 0;
        float S[NB];
#pragma unroll
        for (int n = 0; n < NB; ++n) S[n] = acc[n];
#pragma unroll
        for (int d = 1; d < G; d <<= 1) {
            float So[NB];
#pragma unroll
            for (int n = 0; n < NB; ++n) So[n] = __shfl_up(S[n], d * BT, kWave);
            const int fo = __shfl_up(f, d * BT, kWave);
            if (g >= d) {
                if (!f) {
#pragma unroll
                    for (int n = 0; n < NB; ++n) S[n] += So[n];
                }
                f |= fo;
            }
        }
        if (!f) {
#pragma unroll
            for (int n = 0; n < NB; ++n) S[n] += carry[n];
        }
        float Sp[NB];
#pragma unroll
        for (int n = 0; n < NB; ++n) Sp[n] = __shfl_up(S[n], BT, kWave);
        const int32_t next_head = __shfl_down(head_key, BT, kWave);

        if (multi) {
            const bool take = (ptail == head_key);
            float h[NB];
#pragma unroll
            for (int n = 0; n < NB; ++n) h[n] = head[n] + (take ? (g > 0 ? Sp[n] : carry[n]) : 0.0f);
            write_row(head_key, h);
        }
        if (g < G - 1 && next_head != tail_key) write_row(tail_key, S);

#pragma unroll
        for (int n = 0; n < NB; ++n) carry[n] = __shfl(S[n], (G - 1) * BT + bl, kWave);
        carry_key = __shfl(tail_key, kWave - 1, kWave);
    }
    if (g == 0) write_row(carry_key, carry);
}

// dW[k] = sum_b dyt[r_k, b] * xt[c_k, b]; group g of a wave step takes U
// consecutive slots, its BT lanes split the batch and are reduced by a
// butterfly within the group.
template <int BT, int NB, int U>
__global__ void __launch_bounds__(kBlock) sddmm_kernel(const int32_t* __restrict__ rows,
                                                       const int32_t* __restrict__ cols, int64_t nnz,
                                                       const float* __restrict__ xt, const float* __restrict__ dyt,
                                                       int bp, int ntiles, float* __restrict__ dW, int64_t nsteps)
{
    constexpr int G = kWave / BT;
    constexpr int STEP = G * U;
    const int lane = threadIdx.x & (kWave - 1);
    const int g = lane / BT;
    const int bl = lane - g * BT;
    const int64_t nwaves = (int64_t)gridDim.x * kWavesPerBlock;
    const int bid = (int)blockIdx.x;
    const int per_xcd = (int)((gridDim.x + kXcd - 1) / kXcd);
    const int64_t vb = (int64_t)(bid % kXcd) * per_xcd + bid / kXcd;
    for (int64_t st = vb * kWavesPerBlock + threadIdx.x / kWave; st < nsteps; st += nwaves) {
        const int64_t my = st * STEP + (int64_t)g * U;
        int32_t r[U], c[U];
#pragma unroll
        for (int q = 0; q < U / 4; ++q) {
            const int4 rr = *reinterpret_cast<const int4*>(rows + my + 4 * q);
            const int4 cc = *reinterpret_cast<const int4*>(cols + my + 4 * q);
            r[4 * q + 0] = rr.x; r[4 * q + 1] = rr.y; r[4 * q + 2] = rr.z; r[4 * q + 3] = rr.w;
            c[4 * q + 0] = cc.x; c[4 * q + 1] = cc.y; c[4 * q + 2] = cc.z; c[4 * q + 3] = cc.w;
        }
#pragma unroll
        for (int u = 0; u < U; ++u) {
            if (my + u >= nnz) { r[u] = 0; c[u] = 0; }
        }
        float acc[U];
#pragma unroll
        for (int u = 0; u < U; ++u) acc[u] = 0.0f;
        for (int t = 0; t < ntiles; ++t) {
            const int bc = t * (BT * NB) + bl * NB;
#pragma unroll
            for (int u = 0; u < U; ++u) {
                float x[NB], y[NB];
                load_nb<NB>(xt + (int64_t)c[u] * bp + bc, x);
                load_nb<NB>(dyt + (int64_t)r[u] * bp + bc, y);
#pragma unroll
                for (int n = 0; n < NB; ++n) acc[u] = fmaf(y[n], x[n], acc[u]);
            }
        }
#pragma unroll
        for (int m = BT / 2; m >= 1; m >>= 1) {
#pragma unroll
            for (int u = 0; u < U; ++u) acc[u] += __shfl_xor(acc[u], m, kWave);
        }
        if constexpr (BT == 1) {
            if (my + U <= nnz) {
#pragma unroll
                for (int q = 0; q < U / 4; ++q)
                    *reinterpret_cast<float4*>(dW + my + 4 * q) =
                        make_float4(acc[4 * q], acc[4 * q + 1], acc[4 * q + 2], acc[4 * q + 3]);
            } else {
#pragma unroll
                for (int u = 0; u < U; ++u)
                    if (my + u < nnz) dW[my + u] = acc[u];
            }
        } else {
#pragma unroll
            for (int u = 0; u < U; ++u)
                if ((u % BT) == bl && my + u < nnz) dW[my + u] = acc[u];
        }
    }
}

template <int BT, int NB, int U>
snack_status launch_spmm(const View& v, const float* feat, const BatchPlan& p, int B, float* out, hipStream_t s)
{
    const int nblocks = (v.nchunks + kWavesPerBlock - 1) / kWavesPerBlock;
    const int per_xcd = (nblocks + kXcd - 1) / kXcd;
    dim3 grid((unsigned)(per_xcd * kXcd), (unsigned)p.ntiles);
    hipLaunchKernelGGL((spmm_seg_kernel<BT, NB, U>), grid, dim3(kBlock), 0, s, v.keys, v.idx, v.vals, v.ptr,
                       v.chunk_key, v.nchunks, feat, p.bp, B, v.nkeys, out, per_xcd, nblocks);
    SNACK_HIP(hipGetLastError());
    return SNACK_OK;
}

template <int BT, int NB, int U>
snack_status launch_sddmm(const snack_layer* L, const float* xt, const float* dyt, const BatchPlan& p, float* dW,
                          hipStream_t s)
{
    constexpr int STEP = (kWave / BT) * U;
    const int64_t nsteps = (L->nnz + STEP - 1) / STEP;
    int64_t nb = (nsteps + kWavesPerBlock - 1) / kWavesPerBlock;
    const int64_t cap = 256 * 8 * 4;   // enough resident blocks for the whole chip
    if (nb > cap) nb = cap;
    nb = ((nb + kXcd - 1) / kXcd) * kXcd;
    hipLaunchKernelGGL((sddmm_kernel<BT, NB, U>), dim3((unsigned)nb), dim3(kBlock), 0, s, L->rows, L->cols, L->nnz,
                       xt, dyt, p.bp, p.ntiles, dW, nsteps);
    SNACK_HIP(hipGetLastError());
    return SNACK_OK;
}

}  // namespace

BatchPlan plan_batch(int B)
{
    BatchPlan p;
    if (B <= 1) { p.bt = 1; p.nb = 1; p.u = 4; }
    else if (B == 2) { p.bt = 1; p.nb = 2; p.u = 4; }
    else if (B <= 4) { p.bt = 1; p.nb = 4; p.u = 4; }
    else if (B <= 8) { p.bt = 2; p.nb = 4; p.u = 4; }
    else if (B <= 16) { p.bt = 4; p.nb = 4; p.u = 8; }
    else if (B <= 32) { p.bt = 8; p.nb = 4; p.u = 8; }
    else { p.bt = 16; p.nb = 4; p.u = 16; }
    p.btile = p.bt * p.nb;
    p.ntiles = (B + p.btile - 1) / p.btile;
    p.bp = p.ntiles * p.btile;
    return p;
}

snack_status spmm_view(const View& v, const float* feat_t, const BatchPlan& p, int B, float* out, int kclass,
                       hipStream_t s)
{
    ProfScope prof(kclass, s);
    switch (p.btile) {
    case 1: return launch_spmm<1, 1, 4>(v, feat_t, p, B, out, s);
    case 2: return launch_spmm<1, 2, 4>(v, feat_t, p, B, out, s);
    case 4: return launch_spmm<1, 4, 4>(v, feat_t, p, B, out, s);
    case 8: return launch_spmm<2, 4, 4>(v, feat_t, p, B, out, s);
    case 16: return launch_spmm<4, 4, 8>(v, feat_t, p, B, out, s);
    case 32: return launch_spmm<8, 4, 8>(v, feat_t, p, B, out, s);
    case 64: return launch_spmm<16, 4, 16>(v, feat_t, p, B, out, s);
    default: return SNACK_ERR_INVALID_ARG;
    }
}

snack_status sddmm_dw(const snack_layer* L, const float* xt, const float* dyt, const BatchPlan& p, int B, float* dW,
                      hipStream_t s)
{
    (void)B;
    if (L->nnz == 0) return SNACK_OK;
    ProfScope prof(KC_SDDMM_DW, s);
    switch (p.btile) {
    case 1: return launch_sddmm<1, 1, 4>(L, xt, dyt, p, dW, s);
    case 2: return launch_sddmm<1, 2, 4>(L, xt, dyt, p, dW, s);
    case 4: return launch_sddmm<1, 4, 4>(L, xt, dyt, p, dW, s);
    case 8: return launch_sddmm<2, 4, 4>(L, xt, dyt, p, dW, s);
    case 16: return launch_sddmm<4, 4, 8>(L, xt, dyt, p, dW, s);
    case 32: return launch_sddmm<8, 4, 8>(L, xt, dyt, p, dW, s);
    case 64: return launch_sddmm<16, 4, 16>(L, xt, dyt, p, dW, s);
    default: return SNACK_ERR_INVALID_ARG;
    }
}

}  // namespace snack
