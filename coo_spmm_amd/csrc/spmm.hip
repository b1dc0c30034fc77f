// spmm.hip -- segmented SpMM over a sorted view of the COO triple, fused with
// the sampled dense-dense product for dW.
//
// Forward (SNACK paper, Figure 1; "Padded-CSR" section 6.1) and the input
// gradient ("Padded-CSR" section 7.1, run over the transposed view of section
// 7.2) are one kernel: out[b, key] = sum over the view's entries of that key of
// v * G[idx, b], for a view sorted by key.  The same pass can produce the
// weight gradient on the support ("Padded-CSR" 7.1; SNACK Figure 1's sparse
// outer product): dw[j] = sum_b G[idx_j, b] * H[key_j, b].
//
// Mapping -- one wavefront per key-aligned chunk of the view:
//  * a wave step covers a block of E = 256*P consecutive entries; every lane
//    loads 4P of them with 16-byte loads (the block is read once, coalesced);
//  * the wave is G = 64/BT lane groups; each lane owns NB consecutive batch
//    columns, so a group covers a batch tile of BT*NB columns; the block is
//    split into G contiguous runs, one per group; with BT > 1 the runs reach the
//    group's lanes through LDS, so no index byte is fetched twice from memory;
//  * activations are feature-major (G[idx * bp + b]): the NB values a lane
//    needs per entry are one or two 16-byte loads;
//  * a lane sums its run sequentially per key (head / middle keys / tail);
//    the groups then combine run tails with a segmented Hillis-Steele scan over
//    wavefront shuffles; a key still open at the end of a step is carried into
//    the next.  Every output row is written once, by plain stores: no atomics,
//    so results are bit-reproducible;
//  * the next block is prefetched into registers while the current one is
//    processed.
// Chunks never split a key, so no cross-wave fix-up exists.  Workgroups are
// remapped so each XCD streams one contiguous range of chunks.
//
// dW partial sums are reduced over a group's lanes by one routine
// (reduce4_group) whatever the view, so dW computed over the column view and
// over the row view are bit-identical -- the layer relies on this to update
// its two value copies with streaming SGD.
#include "internal.h"

#include <limits.h>

#include <type_traits>

namespace snack {
namespace {

constexpr int kBlock = 256;
constexpr int kWavesPerBlock = kBlock / kWave;
constexpr int kXcd = 8;

struct RoleArgs {
    const int32_t* idx;
    const uint16_t* idx16;   // the same indices in 16 bits, or null
    const uint16_t* vals16;  // the values rounded to bf16 (inference forward), or null
    int act;                 // activation applied to the outputs as they are stored (inference forward)
    const float* vals;
    const int32_t* ptr;
    const int2* desc;
    const int32_t* empty_keys;
    const int32_t* n_empty;
    const float* G;      // gathered by idx: [nidx, bp]
    const float* H;      // indexed by key: [nkeys, bp] (dW only)
    float* out;          // [B, nkeys] or null
    float* dwo;          // dW in this view's slot order, or null
    float* apply;        // values in this view's slot order to take an SGD step with dW, or null
    float lr;            // (the step uses the entry values the pass loads)
    // with dyo: the MSE gradient of the output written beside it, dyo = mse_scale * (out - tgt)
    // (batch-major like out), and where dyto is set also feature-major [nkeys][bp] (zero past B)
    const float* tgt;
    float* dyo;
    float* dyto;
    float mse_scale;
    int64_t cap;         // padded length of idx / vals
    int32_t nchunks;
    int32_t nkeys;
    int32_t nidx;
    int32_t nblocks;
    int32_t per_xcd;
};

template <int NB>
__device__ inline void load_nb(const float* __restrict__ p, float (&x)[NB])
{
    if constexpr (NB == 8) {
        const float4 a = *reinterpret_cast<const float4*>(p);
        const float4 b = *reinterpret_cast<const float4*>(p + 4);
        x[0] = a.x; x[1] = a.y; x[2] = a.z; x[3] = a.w;
        x[4] = b.x; x[5] = b.y; x[6] = b.z; x[7] = b.w;
    } else if constexpr (NB == 4) {
        const float4 a = *reinterpret_cast<const float4*>(p);
        x[0] = a.x; x[1] = a.y; x[2] = a.z; x[3] = a.w;
    } else if constexpr (NB == 2) {
        const float2 a = *reinterpret_cast<const float2*>(p);
        x[0] = a.x; x[1] = a.y;
    } else {
        x[0] = *p;
    }
}

// Reduce four per-lane values over the BT lanes of a group (a butterfly whose
// upper levels exchange half of the remaining values).  On return lane bl
// holds the full group sum of value (bl / (BT/4)) & 3 for BT >= 4, of values
// {2*bl, 2*bl+1} for BT == 2 (in d[0], d[1]), and all four for BT == 1.
template <int BT>
__device__ inline void reduce4_group(float (&d)[4], int bl)
{
    if constexpr (BT >= 2) {
        {
            constexpr int m = BT / 2;
            const bool hi = (bl & m) != 0;
            const float s0 = hi ? d[0] : d[2];
            const float s1 = hi ? d[1] : d[3];
            const float r0 = __shfl_xor(s0, m, kWave);
            const float r1 = __shfl_xor(s1, m, kWave);
            const float k0 = hi ? d[2] : d[0];
            const float k1 = hi ? d[3] : d[1];
            d[0] = k0 + r0;
            d[1] = k1 + r1;
        }
        if constexpr (BT >= 4) {
            constexpr int m = BT / 4;
            const bool hi = (bl & m) != 0;
            const float s = hi ? d[0] : d[1];
            const float r = __shfl_xor(s, m, kWave);
            d[0] = (hi ? d[1] : d[0]) + r;
#pragma unroll
            for (int mm = BT / 8; mm >= 1; mm >>= 1) d[0] += __shfl_xor(d[0], mm, kWave);
        }
    }
}

// Keys of a run of ascending entries, derived from the chunk's key pointer
// slice held in LDS: entry k belongs to key r0 + j with slice[j] <= k <
// slice[j+1].  Entries outside [s, e) get -1 (before) or INT_MAX (after).
struct KeyWalk {
    const int32_t* slice;
    int32_t r0;
    int32_t nr;
    int64_t s, e;
    int j;
    int32_t nb;

    __device__ inline void start(int64_t k0, int64_t len)
    {
        const int64_t lo_k = k0 > s ? k0 : s;
        const int64_t hi_k = (k0 + len < e) ? k0 + len : e;
        j = 0;
        nb = 0;
        if (lo_k < hi_k) {
            int lo = 0, hi = nr;
            while (hi - lo > 1) {
                const int mid = (lo + hi) >> 1;
                if (slice[mid] <= lo_k) lo = mid;
                else hi = mid;
            }
            j = lo;
            nb = slice[j + 1];
        }
    }
    __device__ inline int32_t key(int64_t k)
    {
        if (k < s) return -1;
        if (k >= e) return INT_MAX;
        while (k >= nb) {
            ++j;
            nb = slice[j + 1];
        }
        return r0 + j;
    }
};

// Per-wave work on one chunk.  SPMM: accumulate out[b, key]; DW: produce dw
// per entry.  Both are compile-time so no load sits under a runtime branch
// (a conditional load makes the compiler wait for every outstanding load).
template <int BT, int NB, int P, bool DW, bool SPMM>
__device__ __forceinline__ void seg_body(const RoleArgs& A, int c, int wv, int lane, int bp, int B,
                                         int32_t* __restrict__ slice, int4* __restrict__ blk_i,
                                         int4* __restrict__ blk_v, const float* __restrict__ Gm)
{
    constexpr int G = kWave / BT;
    constexpr int E = 256 * P;          // entries per wave step
    constexpr int RUN = E / G;          // entries per group per step
    constexpr int NSB = RUN / 4;        // sub-batches of four entries
    static_assert(RUN % 4 == 0, "runs are read four entries at a time");
    static_assert(BT == 1 || P == 1, "wide batch tiles stage one block at a time");
    static_assert(SPMM || DW, "nothing to do");

    const int g = lane / BT;
    const int bl = lane - g * BT;
    const int2 d0 = A.desc[c];
    const int2 d1 = A.desc[c + 1];
    const int32_t r0 = d0.x, r1 = d1.x;
    const int tile0 = (int)blockIdx.y * (BT * NB);
    const int bcol = tile0 + bl * NB;
    const int nkeys = A.nkeys;
    float* __restrict__ out = A.out;

    auto write_row = [&](int32_t key, const float (&a)[NB]) {
        if (key >= r0 && key < r1) {
#pragma unroll
            for (int n = 0; n < NB; ++n) {
                const int b = bcol + n;
                if (b < B) out[(int64_t)b * nkeys + key] = a[n];
            }
        }
    };

    if constexpr (SPMM) {
        if (g == 0) {
            // keys with no entry produce zeros; the role's waves share the list
            const int32_t ne = *A.n_empty;
            for (int i = c; i < ne; i += A.nchunks) {
                const int32_t key = A.empty_keys[i];
#pragma unroll
                for (int n = 0; n < NB; ++n) {
                    const int b = bcol + n;
                    if (b < B) out[(int64_t)b * nkeys + key] = 0.0f;
                }
            }
        }
    }

    const int64_t s = d0.y;
    const int64_t e = d1.y;
    if (s >= e) return;
    const int64_t base0 = s & ~(int64_t)3;
    const int64_t lim = A.cap - E;      // last block start that stays inside the padded arrays
    const int32_t* __restrict__ idx = A.idx;
    const float* __restrict__ vals = A.vals;
    const float* __restrict__ Hm = A.H;

    // the chunk's key pointer slice: nr + 1 <= kChunkWork + 1 values
    const int nr = r1 - r0;
    for (int i = lane; i <= nr; i += kWave) slice[i] = A.ptr[r0 + i];
    __builtin_amdgcn_wave_barrier();
    KeyWalk walk{slice, r0, nr, s, e, 0, 0};

    int32_t carry_key = -1;
    float carry[NB];
#pragma unroll
    for (int n = 0; n < NB; ++n) carry[n] = 0.0f;

    // ---- per-run state and the work on one sub-batch of four entries ----
    int32_t first_key = -1, cur = -1;
    bool multi = false;
    float acc[NB], head[NB];
    int32_t hkey = -2;
    float hreg[NB];
#pragma unroll
    for (int n = 0; n < NB; ++n) hreg[n] = 0.0f;

    auto run_begin = [&]() {
        first_key = -1;
        cur = -1;
        multi = false;
#pragma unroll
        for (int n = 0; n < NB; ++n) {
            acc[n] = 0.0f;
            head[n] = 0.0f;
        }
    };

    auto sub_batch = [&](int64_t k0, bool first, const float (&vv)[4], const float (&y)[4][NB]) {
        int32_t kk[4];
#pragma unroll
        for (int t = 0; t < 4; ++t) kk[t] = walk.key(k0 + t);
        if (first) {
            first_key = kk[0];
            cur = kk[0];
        }
        if constexpr (SPMM) {
            float v[4];
#pragma unroll
            for (int t = 0; t < 4; ++t) v[t] = (k0 + t >= s && k0 + t < e) ? vv[t] : 0.0f;
            if (kk[0] == cur && kk[3] == cur) {
#pragma unroll
                for (int t = 0; t < 4; ++t)
#pragma unroll
                    for (int n = 0; n < NB; ++n) acc[n] = fmaf(v[t], y[t][n], acc[n]);
            } else {
#pragma unroll
                for (int t = 0; t < 4; ++t) {
                    if (kk[t] != cur) {
                        if (multi) {
                            write_row(cur, acc);   // a key wholly inside this run
                        } else {
#pragma unroll
                            for (int n = 0; n < NB; ++n) head[n] = acc[n];
                            multi = true;
                        }
                        cur = kk[t];
#pragma unroll
                        for (int n = 0; n < NB; ++n) acc[n] = 0.0f;
                    }
#pragma unroll
                    for (int n = 0; n < NB; ++n) acc[n] = fmaf(v[t], y[t][n], acc[n]);
                }
            }
        }
        if constexpr (DW) {
            float d[4];
#pragma unroll
            for (int t = 0; t < 4; ++t) {
                const bool inr = kk[t] >= 0 && kk[t] < nkeys;
                if (inr && kk[t] != hkey) {
                    load_nb<NB>(Hm + (int64_t)kk[t] * bp + bcol, hreg);
                    hkey = kk[t];
                }
                float a = 0.0f;
#pragma unroll
                for (int n = 0; n < NB; ++n) a = fmaf(y[t][n], inr ? hreg[n] : 0.0f, a);
                d[t] = a;
            }
            reduce4_group<BT>(d, bl);
            float* __restrict__ dwo = A.dwo;
            if constexpr (BT == 1) {
                if (k0 >= s && k0 + 3 < e) {
                    *reinterpret_cast<float4*>(dwo + k0) = make_float4(d[0], d[1], d[2], d[3]);
                } else {
#pragma unroll
                    for (int t = 0; t < 4; ++t)
                        if (k0 + t >= s && k0 + t < e) dwo[k0 + t] = d[t];
                }
            } else if constexpr (BT == 2) {
#pragma unroll
                for (int t = 0; t < 2; ++t) {
                    const int64_t k = k0 + 2 * bl + t;
                    if (k >= s && k < e) dwo[k] = d[t];
                }
            } else {
                constexpr int STRIDE = BT / 4;
                if ((bl % STRIDE) == 0) {
                    const int64_t k = k0 + bl / STRIDE;
                    if (k >= s && k < e) dwo[k] = d[0];
                }
            }
        }
    };

    // ---- the groups combine their run tails; the open key is carried ----
    auto finish_step = [&]() {
        const int32_t head_key = first_key;
        const int32_t tail_key = cur;
        // the key carried from the previous step is complete unless this step continues it
        const int32_t step_first = __shfl(head_key, 0, kWave);
        if (g == 0 && carry_key != step_first) write_row(carry_key, carry);

        int32_t ptail = __shfl_up(tail_key, BT, kWave);
        if (g == 0) ptail = carry_key;
        int f = (multi || ptail != tail_key) ? 1 : 0;
        float S[NB];
#pragma unroll
        for (int n = 0; n < NB; ++n) S[n] = acc[n];
#pragma unroll
        for (int dd = 1; dd < G; dd <<= 1) {
            float So[NB];
#pragma unroll
            for (int n = 0; n < NB; ++n) So[n] = __shfl_up(S[n], dd * BT, kWave);
            const int fo = __shfl_up(f, dd * BT, kWave);
            if (g >= dd) {
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
    };

    // Blocks of E entries are loaded into rotating register buffers whose
    // prefetch address is clamped into the padding (never under a branch), so
    // a block's index/value loads stay in flight across the previous step.
    struct Buf {
        int4 i[P];
        float4 v[P];
    };
    auto load_buf = [&](int64_t base, Buf& b) {
        const int64_t o0 = (base < lim ? base : lim) + (BT == 1 ? (int64_t)RUN * lane : (int64_t)4 * lane);
#pragma unroll
        for (int q = 0; q < P; ++q) {
            b.i[q] = *reinterpret_cast<const int4*>(idx + o0 + 4 * q);
            if constexpr (SPMM) b.v[q] = *reinterpret_cast<const float4*>(vals + o0 + 4 * q);
        }
    };

    if constexpr (BT == 1) {
        // Each lane's run is its own 4P entries.  Step i issues the gathers of
        // block i, then the loads of block i+2, then reduces block i.
        auto step = [&](int64_t base, const Buf& cb, Buf& pre) {
            float y[RUN][NB];
#pragma unroll
            for (int q = 0; q < P; ++q) {
                load_nb<NB>(Gm + (int64_t)cb.i[q].x * bp + bcol, y[4 * q + 0]);
                load_nb<NB>(Gm + (int64_t)cb.i[q].y * bp + bcol, y[4 * q + 1]);
                load_nb<NB>(Gm + (int64_t)cb.i[q].z * bp + bcol, y[4 * q + 2]);
                load_nb<NB>(Gm + (int64_t)cb.i[q].w * bp + bcol, y[4 * q + 3]);
            }
            load_buf(base + 2 * E, pre);
            const int64_t k0 = base + (int64_t)RUN * lane;
            walk.start(k0, RUN);
            run_begin();
#pragma unroll
            for (int q = 0; q < P; ++q) {
                float vq[4] = {0.0f, 0.0f, 0.0f, 0.0f};
                if constexpr (SPMM) {
                    vq[0] = cb.v[q].x; vq[1] = cb.v[q].y; vq[2] = cb.v[q].z; vq[3] = cb.v[q].w;
                }
                float yq[4][NB];
#pragma unroll
                for (int t = 0; t < 4; ++t)
#pragma unroll
                    for (int n = 0; n < NB; ++n) yq[t][n] = y[4 * q + t][n];
                sub_batch(k0 + 4 * q, q == 0, vq, yq);
            }
            if constexpr (SPMM) finish_step();
        };
        Buf b0, b1, b2;
        load_buf(base0, b0);
        load_buf(base0 + E, b1);
        for (int64_t base = base0;;) {
            step(base, b0, b2);
            base += E;
            if (base >= e) break;
            step(base, b1, b0);
            base += E;
            if (base >= e) break;
            step(base, b2, b1);
            base += E;
            if (base >= e) break;
        }
    } else {
        // Wide batch tiles: the block is staged in LDS and each group reads its
        // run from there (one memory fetch per entry for the whole tile).  The
        // next block is loaded into the same registers once they are in LDS,
        // after this step's gathers are issued.
        int4 ni;
        float4 nv = make_float4(0.0f, 0.0f, 0.0f, 0.0f);
        {
            const int64_t o = (base0 < lim ? base0 : lim) + 4 * lane;
            ni = *reinterpret_cast<const int4*>(idx + o);
            if constexpr (SPMM) nv = *reinterpret_cast<const float4*>(vals + o);
        }
        for (int64_t base = base0; base < e; base += E) {
            blk_i[lane] = ni;
            if constexpr (SPMM) blk_v[lane] = *reinterpret_cast<const int4*>(&nv);
            __builtin_amdgcn_wave_barrier();
            const int64_t run0 = base + (int64_t)g * RUN;
            walk.start(run0, RUN);
            run_begin();
#pragma unroll 2
            for (int sb = 0; sb < NSB; ++sb) {
                const int4 i4 = blk_i[g * NSB + sb];
                float vq[4] = {0.0f, 0.0f, 0.0f, 0.0f};
                if constexpr (SPMM) {
                    const int4 t4 = blk_v[g * NSB + sb];
                    const float4 v4 = *reinterpret_cast<const float4*>(&t4);
                    vq[0] = v4.x; vq[1] = v4.y; vq[2] = v4.z; vq[3] = v4.w;
                }
                float yq[4][NB];
                load_nb<NB>(Gm + (int64_t)i4.x * bp + bcol, yq[0]);
                load_nb<NB>(Gm + (int64_t)i4.y * bp + bcol, yq[1]);
                load_nb<NB>(Gm + (int64_t)i4.z * bp + bcol, yq[2]);
                load_nb<NB>(Gm + (int64_t)i4.w * bp + bcol, yq[3]);
                sub_batch(run0 + 4 * sb, sb == 0, vq, yq);
            }
            {
                const int64_t nb = base + E;
                const int64_t o = (nb < lim ? nb : lim) + 4 * lane;
                ni = *reinterpret_cast<const int4*>(idx + o);
                if constexpr (SPMM) nv = *reinterpret_cast<const float4*>(vals + o);
            }
            if constexpr (SPMM) finish_step();
            __builtin_amdgcn_wave_barrier();
        }
    }
    if constexpr (SPMM) {
        if (g == 0) write_row(carry_key, carry);
    }
}

template <int BT, int NB, int P, bool DW, int WPB, bool XLDS>
__global__ void __launch_bounds__(WPB * kWave) seg_kernel(RoleArgs ra, RoleArgs rb, int grid_a, int bp, int B)
{
    constexpr int E = 256 * P;
    constexpr int LDS_Q = (BT > 1) ? E / 4 : 1;   // int4 per array per wave
    __shared__ int32_t slice_s[WPB][kChunkWork + 2];
    __shared__ int4 blk_s[WPB][2][LDS_Q];
    extern __shared__ __align__(16) float xs_dyn[];   // the gathered operand, when staged in LDS

    const int lane = threadIdx.x & (kWave - 1);
    const int wv = __builtin_amdgcn_readfirstlane((int)(threadIdx.x / kWave));   // uniform: scalar work below
    int bid = (int)blockIdx.x;
    const bool role_a = bid < grid_a;
    if (!role_a) bid -= grid_a;
    const RoleArgs& A = role_a ? ra : rb;
    const int vb = (bid % kXcd) * A.per_xcd + bid / kXcd;
    if (vb >= A.nblocks) return;
    if constexpr (XLDS) {
        // stage the whole gathered operand [nidx, bp] in LDS once per workgroup
        const int64_t n = (int64_t)A.nidx * bp;
        const int64_t n4 = n / 4;
        for (int64_t i = threadIdx.x; i < n4; i += WPB * kWave)
            reinterpret_cast<float4*>(xs_dyn)[i] = reinterpret_cast<const float4*>(A.G)[i];
        for (int64_t i = n4 * 4 + threadIdx.x; i < n; i += WPB * kWave) xs_dyn[i] = A.G[i];
        __syncthreads();
    }
    const int c = vb * WPB + wv;
    if (c >= A.nchunks) return;
    const float* Gm = XLDS ? xs_dyn : A.G;
    // dW is produced only where a dW output exists (a dX-only pass has none)
    const bool want_dw = DW && A.dwo != nullptr && A.H != nullptr;
    if (role_a && A.out != nullptr) {
        if (want_dw) {
            seg_body<BT, NB, P, DW, true>(A, c, wv, lane, bp, B, slice_s[wv], blk_s[wv][0], blk_s[wv][1], Gm);
        } else {
            seg_body<BT, NB, P, false, true>(A, c, wv, lane, bp, B, slice_s[wv], blk_s[wv][0], blk_s[wv][1], Gm);
        }
    } else if constexpr (DW) {
        if (want_dw && blockIdx.y == 0)
            seg_body<BT, NB, P, true, false>(A, c, wv, lane, bp, B, slice_s[wv], blk_s[wv][0], blk_s[wv][1], Gm);
    }
}

// Key-major variant for views whose keys hold many entries (rows or columns
// of hundreds of entries at the densities of interest).  The wave walks its
// keys in order; group g takes a key's entries g, g+G, g+2G, ..., U of them
// in flight, and accumulates its batch columns in registers; at the key's end
// the group sums are added across groups by a fixed xor-shuffle tree and
// written once.  With DW each entry's dot product over the batch tile is
// reduced over the group's lanes (fixed tree) and stored.  Indices are read
// with clamped, unconditional loads so every load stays in flight.  A key's
// blocks always start at its first entry, so a key's sums do not depend on
// which kernel or wave walked it.
template <int BT, int NB, int U>
struct KeyBlock {
    static constexpr int G = kWave / BT;
    static constexpr int STEP = G * U;
    // with STEP <= 64 lane l loads entry base + l and groups pick theirs by
    // shuffles; with wider steps each lane loads its own U entries
    static constexpr bool SHUF = STEP <= kWave;
    static constexpr int NL = SHUF ? 1 : U;
    int32_t nidx[NL];
    float nval[NL];

    // indices and values of the block at base (entries >= lim clamped)
    template <bool SPMM>
    __device__ inline void load(const int32_t* __restrict__ idx, const float* __restrict__ vals, int32_t base,
                                int32_t lim, int lane, int g)
    {
        const int32_t top = lim > 0 ? lim - 1 : 0;
#pragma unroll
        for (int q = 0; q < NL; ++q) {
            const int32_t k = SHUF ? base + lane : base + q * G + g;
            const int32_t kc = k < lim ? k : top;
            nidx[q] = idx[kc];
            nval[q] = SPMM ? vals[kc] : 0.0f;
        }
    }
    // this lane's U entries of the loaded block
    __device__ inline void take(int32_t (&ii)[U], float (&vv)[U], int g) const
    {
        if constexpr (SHUF) {
#pragma unroll
            for (int u = 0; u < U; ++u) {
                ii[u] = __shfl(nidx[0], u * G + g, kWave);
                vv[u] = __shfl(nval[0], u * G + g, kWave);
            }
        } else {
#pragma unroll
            for (int u = 0; u < U; ++u) {
                ii[u] = nidx[u];
                vv[u] = nval[u];
            }
        }
    }
};

template <int NB, int U>
__device__ inline void key_gather(const float* __restrict__ Gm, const int32_t (&ii)[U], int bp, int bcol,
                                  float (&y)[U][NB])
{
#pragma unroll
    for (int u = 0; u < U; ++u) load_nb<NB>(Gm + (int64_t)ii[u] * bp + bcol, y[u]);
}

template <int BT, int NB, int U>
__device__ inline void key_accumulate(const float (&vv)[U], const float (&y)[U][NB], int32_t base, int32_t p1, int g,
                                      float (&acc)[NB])
{
    constexpr int G = kWave / BT;
#pragma unroll
    for (int u = 0; u < U; ++u) {
        const int32_t k = base + u * G + g;
        const float v = k < p1 ? vv[u] : 0.0f;
#pragma unroll
        for (int n = 0; n < NB; ++n) acc[n] = fmaf(v, y[u][n], acc[n]);
    }
}

// entries' dot products with h, four at a time reduced over the group
// together, stored; an entry's result does not depend on U or on its place
// among the four
// (with `apply`, the entry's value also takes its SGD step, from its value vv)
template <int BT, int NB, int U>
__device__ inline void key_dw(const float (&y)[U][NB], const float (&h)[NB], int32_t base, int32_t p1, int g, int bl,
                              float* __restrict__ dwo, const float (&vv)[U], float* __restrict__ apply, float lr)
{
    static_assert(U % 4 == 0, "dW reduces four entries at a time");
    constexpr int G = kWave / BT;
#pragma unroll
    for (int q = 0; q < U / 4; ++q) {
        const int32_t qb = base + 4 * q * G;
        float d[4];
#pragma unroll
        for (int u = 0; u < 4; ++u) {
            float a = 0.0f;
#pragma unroll
            for (int n = 0; n < NB; ++n) a = fmaf(y[4 * q + u][n], h[n], a);
            d[u] = a;
        }
        reduce4_group<BT>(d, bl);
        if constexpr (BT == 1) {
#pragma unroll
            for (int u = 0; u < 4; ++u) {
                const int32_t k = qb + u * G + g;
                if (k < p1) {
                    if (dwo) dwo[k] = d[u];
                    if (apply) apply[k] = sgd_value(vv[4 * q + u], d[u], lr);
                }
            }
        } else if constexpr (BT == 2) {
#pragma unroll
            for (int t = 0; t < 2; ++t) {
                const int32_t k = qb + (2 * bl + t) * G + g;
                if (k < p1) {
                    if (dwo) dwo[k] = d[t];
                    if (apply) apply[k] = sgd_value(vv[4 * q + 2 * bl + t], d[t], lr);
                }
            }
        } else {
            constexpr int STRIDE = BT / 4;
            if ((bl % STRIDE) == 0) {
                const int e = (bl / STRIDE) & 3;
                const int32_t k = qb + e * G + g;
                if (k < p1) {
                    if (dwo) dwo[k] = d[0];
                    if (apply) apply[k] = sgd_value(vv[4 * q + e], d[0], lr);
                }
            }
        }
    }
}

// the MSE targets of key r's NB columns from bcol (clamped, unconditional
// loads: A.tgt is always a valid [B][nkeys] array, the output itself when no
// gradient is written), issued when the key starts so its end does not wait
template <int NB>
__device__ inline void key_targets(const RoleArgs& A, int bcol, int B, int32_t r, float (&tg)[NB])
{
#pragma unroll
    for (int n = 0; n < NB; ++n) tg[n] = A.tgt[(int64_t)(bcol + n < B ? bcol + n : B - 1) * A.nkeys + r];
}

// group sums of a key added across groups, written once by group 0 (with
// A.dyo, the MSE gradient of each written value beside it, from the key's
// targets tg)
template <int BT, int NB>
__device__ inline void key_store(float (&acc)[NB], int g, int bcol, int B, int nkeys, int32_t r, float* __restrict__ out,
                                 const RoleArgs& A, const float (&tg)[NB])
{
#pragma unroll
    for (int m = BT; m < kWave; m <<= 1)
#pragma unroll
        for (int n = 0; n < NB; ++n) acc[n] += __shfl_xor(acc[n], m, kWave);
    if (g == 0) {
#pragma unroll
        for (int n = 0; n < NB; ++n) {
            const int b = bcol + n;
            if (b < B) {
                const int64_t o = (int64_t)b * nkeys + r;
                out[o] = acc[n];
                if (A.dyo) A.dyo[o] = A.mse_scale * (acc[n] - tg[n]);
            }
        }
    }
}

// One chunk's keys; the first block of every key is loaded at the key's start.
// VAL: the entries' values are loaded (always with SPMM; for a dW-only pass,
// where `apply` takes each value's SGD step)
template <int BT, int NB, int U, bool DW, bool SPMM, bool VAL>
__device__ __forceinline__ void key_chunk(const RoleArgs& A, int c, const float* __restrict__ Gm, int bp, int B)
{
    using KB = KeyBlock<BT, NB, U>;
    const int lane = threadIdx.x & (kWave - 1);
    const int g = lane / BT;
    const int bl = lane - g * BT;
    const int2 d0 = A.desc[c];
    const int2 d1 = A.desc[c + 1];
    const int bcol = (int)blockIdx.y * (BT * NB) + bl * NB;
    int32_t p1 = d0.y;
    for (int32_t r = d0.x; r < d1.x; ++r) {
        const int32_t p0 = p1;
        p1 = A.ptr[r + 1];
        float acc[NB];
#pragma unroll
        for (int n = 0; n < NB; ++n) acc[n] = 0.0f;
        float h[NB];
        if constexpr (DW) load_nb<NB>(A.H + (int64_t)r * bp + bcol, h);
        float tg[NB];
        if constexpr (SPMM) key_targets<NB>(A, bcol, B, r, tg);
        KB blk;
        if (p0 < p1) blk.template load<SPMM || VAL>(A.idx, A.vals, p0, p1, lane, g);
        for (int32_t base = p0; base < p1; base += KB::STEP) {
            int32_t ii[U];
            float vv[U];
            blk.take(ii, vv, g);
            float y[U][NB];
            key_gather<NB, U>(Gm, ii, bp, bcol, y);
            blk.template load<SPMM || VAL>(A.idx, A.vals, base + KB::STEP, p1, lane, g);
            if constexpr (SPMM) key_accumulate<BT, NB, U>(vv, y, base, p1, g, acc);
            if constexpr (DW) key_dw<BT, NB, U>(y, h, base, p1, g, bl, A.dwo, vv, A.apply, A.lr);
        }
        if constexpr (SPMM) key_store<BT, NB>(acc, g, bcol, B, A.nkeys, r, A.out, A, tg);
    }
}

__device__ inline int32_t uni(int32_t v) { return (int32_t)__builtin_amdgcn_readfirstlane(v); }

// a key's dW operand: NB batch columns from bcol of row key of a feature-major
// [n][bp] array, or (RM) of column key of a batch-major [B][nkeys] array, the
// columns past B read as zero as in the padded feature-major copy
template <int NB, bool RM>
__device__ inline void load_h(const float* __restrict__ H, int64_t key, int bp, int bcol, int B, int nkeys,
                              float (&h)[NB])
{
    if constexpr (RM) {
        // clamped, unconditional loads; the columns past B zeroed after
        float t[NB];
#pragma unroll
        for (int n = 0; n < NB; ++n) {
            const int b = bcol + n;
            t[n] = H[(int64_t)(b < B ? b : B - 1) * nkeys + key];
        }
#pragma unroll
        for (int n = 0; n < NB; ++n) h[n] = bcol + n < B ? t[n] : 0.0f;
    } else {
        load_nb<NB>(H + key * bp + bcol, h);
    }
}

template <int BT, int NB, int U, bool DW, bool SPMM = true, bool VAL = SPMM>
__global__ void __launch_bounds__(kBlock) key_kernel(RoleArgs A, int bp, int B)
{
    const int bid = (int)blockIdx.x;
    const int vb = (bid % kXcd) * A.per_xcd + bid / kXcd;
    if (vb >= A.nblocks) return;
    const int c = vb * kWavesPerBlock + uni((int)(threadIdx.x / kWave));   // uniform: scalar loads of the chunk
    if (c >= A.nchunks) return;
    key_chunk<BT, NB, U, DW, SPMM, VAL>(A, c, A.G, bp, B);
}

// workgroup size of the streamed kernel (batch tiles 1-4, operand in LDS)
constexpr int kLdsKeyWaves = 16;

// ---- slice-tiled key-major kernel (batch tiles of 16 to 64 columns) --------
// A wide batch makes every entry gather a long operand row (256 bytes at 64
// columns), which the vector caches serve far below LDS rates.  The operand's
// rows are split into S slices that each fit in LDS; workgroup (slice s, key
// block) stages slice s once and its wavefronts walk the segments of their
// keys that fall in it -- every gather is an LDS read of a row laid out so a
// quarter-wave reads 256 contiguous bytes.  Each wavefront streams the blocks
// of its keys' segments with kTileDepth blocks in flight (a ring of statically
// indexed registers, so no in-flight register is ever copied); the lanes of a
// group receive their entries, and sum across groups, through DPP and lane
// swaps, so the LDS pipe carries nothing but the gathers.  Slice partial
// sums of a key are written to a [S][nkeys][tile] buffer and added in slice
// order by a second kernel: no atomics, results bit-reproducible.  Per-entry
// dW needs no such step (an entry lies in exactly one slice).
constexpr int kTileWaves = 16;
constexpr int kTileDepth = 8;     // blocks in flight per wavefront
constexpr int kTileDepthDw = 4;   // with dW: each block also holds its key's operand row
constexpr int kTileStaticLds = 1024;   // bytes kept back from the slice buffer

struct TileArgs {
    const int32_t* tab;   // slice bounds of key r in slice s: tab[s * tstride + r], tab[(s + 1) * tstride + r]
    int64_t tstride;
    float* part;          // [S][nkeys][tile] partial sums per batch tile, or null to write the outputs (S == 1)
    int64_t pstride;      // floats between two batch tiles' partial sums
    int64_t dwstride;     // floats between two batch tiles' dW (several tiles: one dW slab per tile)
    int32_t S, KB, R;     // slices, key blocks, keys per block
};

// one block of a key's segment: entries [base, lim) of key r (all uniform);
// an exhausted cursor yields lim = -1 < base = 0 (no entries, no key end).
// The flags are compares of base and lim, so they stay in scalar registers.
struct TileDesc {
    int32_t base, lim, r;
    __device__ inline bool valid() const { return lim >= base; }
    template <int STEP>
    __device__ inline bool last() const { return lim >= base && base + STEP >= lim; }
};

// a wavefront's keys r0, r0 + kTileWaves, ... (nk <= 64 of them); lane j
// holds key j's slice bounds
struct TileCursor {
    int32_t tlo, thi;
    int32_t j, nk, r0, base, p1;

    __device__ inline void next(TileDesc& d, int32_t step)
    {
        if (j >= nk) {
            d.base = 0;
            d.lim = -1;
            d.r = r0;
            return;
        }
        d.base = base;
        d.lim = p1;
        d.r = r0 + kTileWaves * j;
        if (base + step >= p1) {
            ++j;
            if (j < nk) {
                base = uni(__builtin_amdgcn_readlane(tlo, j));
                p1 = uni(__builtin_amdgcn_readlane(thi, j));
            }
        } else {
            base += step;
        }
    }
};

// ---- lane exchanges on the VALU (DPP and gfx950 lane swaps) ---------------
// The tile kernel keeps the LDS pipe for its gathers: every other exchange
// between lanes goes through data-parallel primitives instead of LDS-routed
// shuffles.
template <int CTRL, int BANKS = 0xF>
__device__ inline float dpp_f(float old, float x)
{
    return __int_as_float(__builtin_amdgcn_update_dpp(__float_as_int(old), __float_as_int(x), CTRL, 0xF, BANKS, false));
}
template <int CTRL, int BANKS = 0xF>
__device__ inline int32_t dpp_i(int32_t old, int32_t x)
{
    return __builtin_amdgcn_update_dpp(old, x, CTRL, 0xF, BANKS, false);
}
// x[lane ^ M] for M < 16 (within a row of 16 lanes)
template <int M>
__device__ inline float lane_xor(float x)
{
    static_assert(M == 1 || M == 2 || M == 4 || M == 8, "within a row");
    // every source lane exists for these patterns, so no old value is needed
    // (plain moves, which the compiler folds into the following add)
    if constexpr (M == 1) return __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(x), 0xB1, 0xF, 0xF, true));
    else if constexpr (M == 2) return __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(x), 0x4E, 0xF, 0xF, true));
    else if constexpr (M == 4)   // half-row mirror, then quad reverse (every source lane exists: no old value)
        return dpp_f<0x1B>(0.0f, __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(x), 0x141, 0xF, 0xF, true)));
    else return __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(x), 0x128, 0xF, 0xF, true));   // row ror 8
}
// value of lane U0 of this lane's group of BT lanes (groups are rows, half
// rows or quads)
template <int BT, int U0>
__device__ inline int32_t group_bcast(int32_t x)
{
    if constexpr (BT == 16) return __builtin_amdgcn_mov_dpp(x, 0x150 + U0, 0xF, 0xF, false);   // row broadcast
    else if constexpr (BT == 8) return dpp_i<0x158 + U0, 0xC>(dpp_i<0x150 + U0, 0x3>(x, x), x);
    else if constexpr (BT == 4) return __builtin_amdgcn_mov_dpp(x, U0 * 0x55, 0xF, 0xF, false);   // quad broadcast
    else return __builtin_amdgcn_mov_dpp(x, U0 | (U0 << 2) | ((2 + U0) << 4) | ((2 + U0) << 6), 0xF, 0xF, false);
}
// group_bcast with zero in lanes a masked broadcast leaves untouched; the form
// the compiler folds into a following add
template <int BT, int U0>
__device__ inline int32_t group_bcast0(int32_t x)
{
    if constexpr (BT == 16) return dpp_i<0x150 + U0>(0, x);
    else if constexpr (BT == 8) return dpp_i<0x158 + U0, 0xC>(dpp_i<0x150 + U0, 0x3>(0, x), x);
    else if constexpr (BT == 4) return dpp_i<U0 * 0x55>(0, x);
    else return dpp_i<U0 | (U0 << 2) | ((2 + U0) << 4) | ((2 + U0) << 6)>(0, x);   // pair broadcast
}
// one exchange-halves level over lane bit BIT on the first CNT values: the
// lanes with the bit clear end with value i summed over both halves in a[i],
// the others with value i + CNT / 2.  Across bits 5 and 4 one lane swap of the
// pair does the exchange (the swap leaves value i of both halves in one
// register and value i + CNT / 2 of both in the other, each in the lanes that
// keep it); lower bits select what to send and take the partner's by DPP.
template <int BIT, int CNT, int NB>
__device__ inline void xlevel(float (&a)[NB], int lane)
{
    if constexpr (BIT >= 4) {
#pragma unroll
        for (int i = 0; i < CNT / 2; ++i) {
            const auto r = BIT == 5 ? __builtin_amdgcn_permlane32_swap(__float_as_uint(a[i]),
                                                                       __float_as_uint(a[i + CNT / 2]), false, false)
                                    : __builtin_amdgcn_permlane16_swap(__float_as_uint(a[i]),
                                                                       __float_as_uint(a[i + CNT / 2]), false, false);
            a[i] = __uint_as_float(r[0]) + __uint_as_float(r[1]);
        }
    } else {
        const bool hi = ((lane >> BIT) & 1) != 0;
#pragma unroll
        for (int i = 0; i < CNT / 2; ++i) {
            const float sv = hi ? a[i] : a[i + CNT / 2];
            const float kv = hi ? a[i + CNT / 2] : a[i];
            a[i] = kv + lane_xor<(1 << BIT)>(sv);
        }
    }
}
// NB values (4 or 8) summed over the G = 64 / BT groups of a wave: exchange
// halves over the top log2(NB) lane bits, then plain sums over the remaining
// group bits.  Lane l ends with the total of value v = (l >> (6 - log2 NB)), the
// value's column being 4 * (l % BT + BT * (v >> 2)) + (v & 3); lanes that
// differ only in the plain-summed bits hold the same total.
template <int BT, int NB>
__device__ inline float group_reduce(float (&a)[NB], int lane)
{
    static_assert(NB == 4 || NB == 8, "four or eight values per lane");
    static_assert(64 / BT >= NB, "at least one group per value");
    xlevel<5, NB>(a, lane);
    xlevel<4, NB / 2>(a, lane);
    if constexpr (NB == 8) xlevel<3, 2>(a, lane);
    float c = a[0];
    constexpr int LOWX = NB == 8 ? 3 : 4;   // lowest exchanged lane bit
    if constexpr (LOWX > 3 && BT <= 8) c += lane_xor<8>(c);   // lane bit 3 is a group bit
    if constexpr (BT <= 4) c += lane_xor<4>(c);               // bit 2
    if constexpr (BT <= 2) c += lane_xor<2>(c);               // bit 1
    if constexpr (BT <= 1) c += lane_xor<1>(c);               // bit 0
    return c;
}
template <int BT, int NB>
__device__ inline int group_reduce_col(int lane)
{
    constexpr int SH = NB == 8 ? 3 : 4;
    const int v = lane >> SH;
    return 4 * ((lane % BT) + BT * (v >> 2)) + (v & 3);
}
template <int BT, int NB>
__device__ inline bool group_reduce_owner(int lane)
{
    constexpr int SH = NB == 8 ? 3 : 4;
    return (lane & ((1 << SH) - 1) & ~(BT - 1)) == 0;
}

// reduce4_group with its exchanges on the VALU (groups of 4, 8 or 16 lanes)
template <int BT>
__device__ inline void reduce4_dpp(float (&d)[4], int bl)
{
    static_assert(BT >= 4 && BT <= 16, "groups of 4 to 16 lanes");
    {
        constexpr int m = BT / 2;
        const bool hi = (bl & m) != 0;
        const float s0 = hi ? d[0] : d[2];
        const float s1 = hi ? d[1] : d[3];
        const float r0 = lane_xor<m>(s0);
        const float r1 = lane_xor<m>(s1);
        d[0] = (hi ? d[2] : d[0]) + r0;
        d[1] = (hi ? d[3] : d[1]) + r1;
    }
    {
        constexpr int m = BT / 4;
        const bool hi = (bl & m) != 0;
        const float sv = hi ? d[0] : d[1];
        const float r = lane_xor<m>(sv);
        d[0] = (hi ? d[1] : d[0]) + r;
    }
    if constexpr (BT >= 16) d[0] += lane_xor<2>(d[0]);
    if constexpr (BT >= 8) d[0] += lane_xor<1>(d[0]);
}

// A block of the tile kernel: group g owns entries base + g*U + u (u < U);
// lane bl of the group loads entry bl / (BT / U) (clamped, unconditional loads
// keep every block in flight; the lane that ends up owning an entry's reduced
// dW is one that loaded it), and the group's lanes get each entry by a broadcast
// inside the group.  Before use, entries outside [base, lim) are neutralised
// per lane -- value 0 and an all-zero row staged after the slice -- so the
// per-entry work needs no masks, and the index becomes the entry's byte offset
// into the slice.
template <int BT, int U>
struct TileBlock {
    static constexpr int G = kWave / BT;
    static constexpr int STEP = G * U;
    static constexpr int LS = BT / U;   // lanes per loaded entry
    static_assert(U <= BT && (U % 2) == 0 && BT % U == 0, "a group's lanes load its entries");
    int32_t nidx;
    float nval;
    int32_t noff;
    float mval;

    // lk = g * U + bl / LS: the lane's entry within the block.  The block's
    // base pointers are uniform, so the per-lane part is a small byte offset.
    template <bool SPMM>
    __device__ inline void load(const int32_t* __restrict__ idx, const float* __restrict__ vals, int32_t base,
                                int32_t lim, int32_t lk)
    {
        const int32_t span = lim - base;
        const uint32_t ob = (uint32_t)min(lk, span > 0 ? span - 1 : 0) * 4u;
        nidx = *reinterpret_cast<const int32_t*>(reinterpret_cast<const char*>(idx + base) + ob);
        nval = SPMM ? *reinterpret_cast<const float*>(reinterpret_cast<const char*>(vals + base) + ob) : 0.0f;
    }
    // zero_off: the all-zero row staged after the slice, so a neutral entry
    // adds exactly 0 whatever the activations hold
    __device__ inline void prepare(int32_t base, int32_t lim, int32_t lk, int32_t i0, int32_t row_bytes,
                                   int32_t zero_off)
    {
        const bool in = lk < lim - base;
        noff = in ? (nidx - i0) * row_bytes : zero_off;
        mval = in ? nval : 0.0f;
    }
    // entry u's offset plus this lane's column offset (the broadcast folds
    // into the add), and its value
    template <int U0>
    __device__ inline int32_t off_at(int32_t lane_off) const
    {
        return group_bcast0<BT, U0 * LS>(noff) + lane_off;
    }
    template <int U0>
    __device__ inline float val_at() const
    {
        return __int_as_float(group_bcast<BT, U0 * LS>(__float_as_int(mval)));
    }
};

// the U entries' staged rows -- NB floats of this lane each: 16-byte chunk
// lane % BT of the row, and for NB = 8 also chunk lane % BT + BT -- and values
template <int U, int BT, int NB, int U0 = 0, class TB>
__device__ inline void tile_gather(const TB& b, int32_t lane_off, float (&y)[U][NB])
{
    extern __shared__ __align__(16) float gs_dyn[];
    if constexpr (U0 < U) {
        const int32_t off = b.template off_at<U0>(lane_off);
        const char* base = reinterpret_cast<const char*>(gs_dyn) + off;
        const float4 v = *reinterpret_cast<const float4*>(base);
        y[U0][0] = v.x;
        y[U0][1] = v.y;
        y[U0][2] = v.z;
        y[U0][3] = v.w;
        if constexpr (NB == 8) {
            const float4 w = *reinterpret_cast<const float4*>(base + BT * 16);
            y[U0][4] = w.x;
            y[U0][5] = w.y;
            y[U0][6] = w.z;
            y[U0][7] = w.w;
        }
        tile_gather<U, BT, NB, U0 + 1>(b, lane_off, y);
    }
}
template <int U, int U0 = 0, class TB>
__device__ inline void tile_vals(const TB& b, float (&vv)[U])
{
    if constexpr (U0 < U) {
        vv[U0] = b.template val_at<U0>();
        tile_vals<U, U0 + 1>(b, vv);
    }
}

// element i (0 <= i < 2^30) of an array whose base is uniform: a small
// per-lane byte offset on a scalar base
__device__ inline float* lane_at(float* base, int32_t i)
{
    return reinterpret_cast<float*>(reinterpret_cast<char*>(base) + (uint32_t)i * 4u);
}

// per-entry dot products with the key's operand row, reduced over the group
// (pairs for 2-lane groups, fours otherwise) and stored; an entry's result is
// the same sum of the same per-lane partials as in the key-major kernels.
// The lane left holding entry e's sum is one that loaded entry e (lk, value
// own), so with `apply` the value takes its SGD step without a lane exchange.
template <int BT, int NB, int U>
__device__ inline void tile_dw(const float (&y)[U][NB], const float (&h)[NB], int32_t base, int32_t lim, int32_t lk,
                               int bl, float* __restrict__ dwo, float own, float* __restrict__ apply, float lr)
{
    static_assert((BT == 2 && U == 2) || (BT >= 4 && U == 4), "owner lanes are loader lanes");
    if constexpr (BT == 2) {
#pragma unroll
        for (int q = 0; q < U / 2; ++q) {
            float d[2];
#pragma unroll
            for (int t = 0; t < 2; ++t) {
                float a = 0.0f;
#pragma unroll
                for (int n = 0; n < NB; ++n) a = fmaf(y[2 * q + t][n], h[n], a);
                d[t] = a;
            }
            const bool hi = (bl & 1) != 0;
            const float r = lane_xor<1>(hi ? d[0] : d[1]);
            const float tot = (hi ? d[1] : d[0]) + r;
            if (lk < lim - base) {
                if (dwo) *lane_at(dwo + base, lk) = tot;
                if (apply) *lane_at(apply + base, lk) = sgd_value(own, tot, lr);
            }
        }
    } else {
        constexpr int STRIDE = BT / 4;
#pragma unroll
        for (int q = 0; q < U / 4; ++q) {
            float d[4];
#pragma unroll
            for (int t = 0; t < 4; ++t) {
                float a = 0.0f;
#pragma unroll
                for (int n = 0; n < NB; ++n) a = fmaf(y[4 * q + t][n], h[n], a);
                d[t] = a;
            }
            reduce4_dpp<BT>(d, bl);
            // lane bl holds entry bl / STRIDE, the entry it loaded
            if ((bl % STRIDE) == 0 && lk < lim - base) {
                if (dwo) *lane_at(dwo + base, lk) = d[0];
                if (apply) *lane_at(apply + base, lk) = sgd_value(own, d[0], lr);
            }
        }
    }
}

// the key's dW operand: the lane's NB columns of row key of a feature-major array
template <int BT, int NB>
__device__ inline void tile_h(const float* __restrict__ H, int64_t key, int bp, int32_t lane_off, float (&h)[NB])
{
    const float* p = reinterpret_cast<const float*>(reinterpret_cast<const char*>(H + key * bp) + (uint32_t)lane_off);
    const float4 a = *reinterpret_cast<const float4*>(p);
    h[0] = a.x;
    h[1] = a.y;
    h[2] = a.z;
    h[3] = a.w;
    if constexpr (NB == 8) {
        const float4 b = *reinterpret_cast<const float4*>(p + 4 * BT);
        h[4] = b.x;
        h[5] = b.y;
        h[6] = b.z;
        h[7] = b.w;
    }
}

// The slice-tiled pass of one workgroup: `bid` of `nwg` workgroups of the role
// (a multiple of kXcd), over batch tile `tile`.
template <int BT, int NB, int U, int D, bool DW, bool SPMM, bool VAL = SPMM>
__device__ __forceinline__ void tile_body(RoleArgs A, const TileArgs& T, int bp, int B, int bid, int nwg, int tile)
{
    constexpr int BTILE = BT * NB;
    constexpr int ROW = tile_row_floats(BTILE);   // floats per staged row
    using TB = TileBlock<BT, U>;
    extern __shared__ __align__(16) float gs_dyn[];
    const int per = nwg / kXcd;   // the grid is a multiple of kXcd
    // workgroups of one XCD take consecutive (slice, key block) pairs: they share slices in L2
    const int lg = (bid % kXcd) * per + bid / kXcd;
    const int s = lg / T.KB;
    const int kb = lg - s * T.KB;
    if (s >= T.S) return;
    const int nkeys = A.nkeys;
    // batch tile (grid dimension y); over several tiles, a dW pass reads the
    // tile's columns of the key's row and writes the tile's own dW slab
    if constexpr (DW) {
        A.H += (int64_t)tile * BTILE;
        A.dwo += (int64_t)tile * T.dwstride;
    }
    const int32_t i0 = split_start(s, T.S, A.nidx);
    const int32_t nrow = split_start(s + 1, T.S, A.nidx) - i0;
    {
        // the tile's columns of the slice's rows (BTILE floats, bp apart in global memory;
        // contiguous when the batch is a single tile) into LDS rows of ROW floats
        constexpr int Q = BTILE / 4, RQ = ROW / 4;
        const int64_t n4 = (int64_t)nrow * Q;
        const int64_t rs4 = bp / 4;
        const float4* __restrict__ src = reinterpret_cast<const float4*>(A.G + (int64_t)i0 * bp + (int64_t)tile * BTILE);
        float4* dst = reinterpret_cast<float4*>(gs_dyn);
        constexpr int SB = 8;
        constexpr int NT = kTileWaves * kWave;
        for (int64_t q0 = threadIdx.x; q0 < n4; q0 += (int64_t)SB * NT) {
            float4 v[SB];
#pragma unroll
            for (int k = 0; k < SB; ++k) {
                const int64_t q = q0 + (int64_t)k * NT;
                const int64_t qc = q < n4 ? q : n4 - 1;
                v[k] = src[(qc / Q) * rs4 + (qc % Q)];
            }
            // clamped, unconditional stores (tail lanes rewrite the last element
            // with its own value) keep all SB loads in flight together
#pragma unroll
            for (int k = 0; k < SB; ++k) {
                const int64_t q = q0 + (int64_t)k * NT;
                const int64_t qc = q < n4 ? q : n4 - 1;
                dst[(qc / Q) * RQ + (qc % Q)] = v[k];
            }
        }
        if (threadIdx.x < BTILE / 4) dst[(int64_t)nrow * RQ + threadIdx.x] = make_float4(0.0f, 0.0f, 0.0f, 0.0f);   // zero row
        __syncthreads();
    }
    const int lane = threadIdx.x & (kWave - 1);
    const int wv = uni((int)(threadIdx.x / kWave));
    const int g = lane / BT;
    const int bl = lane - g * BT;
    const int32_t rb = kb * T.R;
    const int32_t re = rb + T.R < nkeys ? rb + T.R : nkeys;
    const int32_t r0 = rb + wv;
    const int32_t nk = r0 < re ? (re - r0 + kTileWaves - 1) / kTileWaves : 0;
    if (nk == 0) return;
    TileCursor cur;
    {
        const int32_t rj = r0 + kTileWaves * (lane < nk ? lane : 0);
        cur.tlo = T.tab[(int64_t)s * T.tstride + rj];
        cur.thi = T.tab[(int64_t)(s + 1) * T.tstride + rj];
    }
    cur.j = 0;
    cur.nk = nk;
    cur.r0 = r0;
    cur.base = uni(__builtin_amdgcn_readlane(cur.tlo, 0));
    cur.p1 = uni(__builtin_amdgcn_readlane(cur.thi, 0));

    const int32_t lk = g * U + bl / TB::LS;   // the lane's entry within a block
    const int32_t lane_off = bl * 16;
    TileDesc d[D];
    TB blk[D];
    float hb[D][NB];
#pragma unroll
    for (int q = 0; q < D; ++q) {
        cur.next(d[q], TB::STEP);
        blk[q].template load<SPMM || VAL>(A.idx, A.vals, d[q].base, d[q].lim, lk);
        if constexpr (DW) tile_h<BT, NB>(A.H, d[q].r, bp, lane_off, hb[q]);
    }
    float acc[NB];
#pragma unroll
    for (int n = 0; n < NB; ++n) acc[n] = 0.0f;
    // every slot of a round is processed (an exhausted cursor yields empty,
    // fully masked blocks), so the loop has a single exit and each slot keeps
    // its registers across rounds
    for (;;) {
#pragma unroll
        for (int q = 0; q < D; ++q) {
            blk[q].prepare(d[q].base, d[q].lim, lk, i0, ROW * 4, nrow * ROW * 4);
            float y[U][NB];
            tile_gather<U, BT, NB>(blk[q], lane_off, y);
            if constexpr (SPMM) {
                float vv[U];
                tile_vals<U>(blk[q], vv);
#pragma unroll
                for (int u = 0; u < U; ++u)
#pragma unroll
                    for (int n = 0; n < NB; ++n) acc[n] = fmaf(vv[u], y[u][n], acc[n]);
            }
            if constexpr (DW)
                tile_dw<BT, NB, U>(y, hb[q], d[q].base, d[q].lim, lk, bl, A.dwo, blk[q].mval, A.apply, A.lr);
            if constexpr (SPMM) {
                if (d[q].template last<TB::STEP>()) {
                    // each lane ends with one column of the key's sum; one lane per column stores
                    const float tot = group_reduce<BT, NB>(acc, lane);
                    const int b = group_reduce_col<BT, NB>(lane);
                    if (group_reduce_owner<BT, NB>(lane)) {
                        if (T.part) T.part[tile * T.pstride + ((int64_t)s * nkeys + d[q].r) * BTILE + b] = tot;
                        else if (tile * BTILE + b < B) A.out[(int64_t)(tile * BTILE + b) * nkeys + d[q].r] = tot;
                    }
#pragma unroll
                    for (int n = 0; n < NB; ++n) acc[n] = 0.0f;
                }
            }
            cur.next(d[q], TB::STEP);
            blk[q].template load<SPMM || VAL>(A.idx, A.vals, d[q].base, d[q].lim, lk);
            if constexpr (DW) tile_h<BT, NB>(A.H, d[q].r, bp, lane_off, hb[q]);
        }
        if (!d[0].valid()) break;
    }
}

template <int BT, int NB, int U, int D, bool DW, bool SPMM, bool VAL = SPMM>
__global__ void __launch_bounds__(kTileWaves * kWave) tile_kernel(RoleArgs A, TileArgs T, int bp, int B)
{
    tile_body<BT, NB, U, D, DW, SPMM, VAL>(A, T, bp, B, (int)blockIdx.x, (int)gridDim.x, (int)blockIdx.y);
}

// The backward's two slice-tiled passes of one batch tile in one launch: the
// first g0 workgroups the column pass (dX partial sums; the column-ordered
// values stepped in place from the dW they compute), the rest the row pass
// (dW in canonical order; the canonical values stepped in place).  Neither
// reads what the other writes.
template <int BT, int NB, int U, int D>
__global__ void __launch_bounds__(kTileWaves * kWave)
    tile_bwd_kernel(RoleArgs Ac, TileArgs Tc, RoleArgs Ar, TileArgs Tr, int g0, int bp, int B)
{
    const int bid = (int)blockIdx.x;
    if (bid < g0) tile_body<BT, NB, U, D, true, true, true>(Ac, Tc, bp, B, bid, g0, 0);
    else tile_body<BT, NB, U, D, true, false, true>(Ar, Tr, bp, B, bid - g0, (int)gridDim.x - g0, 0);
}

// ---- streamed kernel for batch tiles of 1 to 4 columns, operand in LDS ----
// At narrow batches every pass is a stream of the view's index and values (8
// bytes per entry) with a handful of instructions per entry, so what bounds it
// is how many bytes each wavefront keeps in flight.  Each lane owns four
// consecutive entries of a 256-entry block (one 16-byte load each for indices
// and values, every block one coalesced kilobyte per array), and a wavefront
// keeps D blocks in flight in a ring of statically indexed registers while it
// works on the oldest.  Blocks never cross a key: a key's blocks start at its
// first entry rounded down to four, so a block's lanes mask the entries
// outside the key (value 0 on an all-zero LDS row past the operand: a masked
// entry adds exactly 0 whatever the activations hold).  A lane owns every
// batch column of its entries, so the dW of an entry is one fused multiply-add
// chain over the columns in order -- the same arithmetic as every other
// one-lane-per-tile kernel here, so the row and column views give bit-identical
// dW.  Key sums are added over the wavefront by a fixed tree when the key's
// last block is done and stored once: no atomics, bit-reproducible.  The
// grid is persistent (every workgroup stages the operand once); wavefront w of
// W takes the keys [nkeys w / W, nkeys (w+1) / W), whose pointer it reads as a
// window across its lanes, so every block address follows from registers
// (supports drawn uniformly give every key about the same length, hence every
// wavefront about the same work).  The operand's staging loads, and then the
// first D blocks, are issued before anything waits on them.
constexpr int kStreamBlock = 256;   // entries per block: 4 per lane

// one block: the entries [base, base + 256) of key r that lie in [lo, hi);
// flags bit 0: the key's first block, bit 1: its last.  hi < lo: no block
// (an exhausted cursor), which touches nothing.  All fields wave-uniform.
struct StreamDesc {
    int32_t base, lo, hi, r, flags;
    __device__ inline bool valid() const { return hi >= lo; }
};

// A wavefront's keys [ra, rb), walked block by block.  The key pointer of up
// to 64 keys at a time sits in a register across the lanes (lane j holds
// ptr[wb + j]), so producing the next block needs no memory access except a
// reload after every 63 keys.
struct StreamCursor {
    const int32_t* ptr;
    int32_t nkeys;
    int32_t rb;          // end of the wavefront's keys
    int32_t wb, j;       // window base key, current key wb + j
    int32_t win;         // this lane's ptr[min(wb + lane, nkeys)]
    int32_t p0, p1, base;
    bool done;

    __device__ inline void load_window(int lane)
    {
        const int32_t k = wb + lane;
        win = ptr[k < nkeys ? k : nkeys];
    }
    __device__ inline void start(int32_t ra, int32_t rend, int lane)
    {
        rb = rend;
        wb = ra;
        j = 0;
        done = ra >= rend;
        load_window(lane);
        p0 = uni(__builtin_amdgcn_readlane(win, 0));
        p1 = uni(__builtin_amdgcn_readlane(win, 1));
        base = p0 & ~3;
    }
    __device__ inline void next(StreamDesc& d, int lane)
    {
        if (done) {
            d.base = 0;
            d.lo = 1;
            d.hi = 0;
            d.r = 0;
            d.flags = 0;
            return;
        }
        d.base = base;
        d.lo = p0;
        d.hi = p1;
        d.r = wb + j;
        int f = base == (p0 & ~3) ? 1 : 0;
        if (base + kStreamBlock >= p1) {
            f |= 2;
            if (wb + j + 1 >= rb) {
                done = true;
            } else {
                // the reloaded window is read inside its own branch, so the wait
                // for that load stays there and the common path waits on nothing
                int32_t np1;
                if (j + 1 == kWave - 1) {
                    wb += kWave - 1;
                    j = 0;
                    load_window(lane);
                    np1 = uni(__builtin_amdgcn_readlane(win, 1));
                } else {
                    ++j;
                    np1 = uni(__builtin_amdgcn_readlane(win, j + 1));
                }
                p0 = p1;
                p1 = np1;
                base = p0 & ~3;
            }
        } else {
            base += kStreamBlock;
        }
        d.flags = f;
    }
};

// x summed over the 64 lanes of the wavefront by a fixed tree (every lane ends
// with the total)
__device__ inline float wave_sum(float x)
{
    x += lane_xor<1>(x);
    x += lane_xor<2>(x);
    x += lane_xor<4>(x);
    x += lane_xor<8>(x);
    x += __shfl_xor(x, 16, kWave);
    x += __shfl_xor(x, 32, kWave);
    return x;
}

template <int NB>
__device__ inline void lds_row(const float* __restrict__ g, int32_t i, float (&y)[NB])
{
    if constexpr (NB == 4) {
        const float4 a = reinterpret_cast<const float4*>(g)[i];
        y[0] = a.x; y[1] = a.y; y[2] = a.z; y[3] = a.w;
    } else if constexpr (NB == 2) {
        const float2 a = reinterpret_cast<const float2*>(g)[i];
        y[0] = a.x; y[1] = a.y;
    } else {
        y[0] = g[i];
    }
}

// The operand [nidx][NB] (feature-major, the row of feature i at i * NB) staged
// into LDS by the streamed kernel's 1024 threads: load() issues every load of a
// thread's share (at most 10 rows of 16 bytes: LDS holds at most 160 KB), and
// store() writes them.  With RM the source is the caller's batch-major
// [B][nidx] array, read as 16-byte runs of four features per batch row and
// transposed in registers; batch columns past B are zero, as in the padded
// feature-major copy.  Sources that are not 16-byte aligned or whose rows are
// not a multiple of four floats take a plain loop in store().
template <int NB, bool RM>
struct StreamStage {
    static constexpr int NT = kLdsKeyWaves * kWave;
    static constexpr int QU = RM ? (10 + NB - 1) / NB : 10;   // 16-byte loads per batch row and thread
    float4 v[QU][RM ? NB : 1];
    bool vec;

    __device__ inline void load(const float* __restrict__ G, int nidx, int B)
    {
        const int tid = threadIdx.x;
        if constexpr (RM) {
            vec = (nidx % 4) == 0 && (reinterpret_cast<uintptr_t>(G) & 15) == 0;
            const int n4 = vec ? nidx / 4 : 0;
#pragma unroll
            for (int u = 0; u < QU; ++u) {
                const int q = tid + u * NT;
                const int qc = q < n4 ? q : (n4 > 0 ? n4 - 1 : 0);
#pragma unroll
                for (int b = 0; b < NB; ++b)
                    v[u][b] = n4 > 0 ? reinterpret_cast<const float4*>(G + (int64_t)(b < B ? b : B - 1) * nidx)[qc]
                                     : make_float4(0.0f, 0.0f, 0.0f, 0.0f);
            }
        } else {
            const int n = nidx * NB;
            vec = (n % 4) == 0 && (reinterpret_cast<uintptr_t>(G) & 15) == 0;
            const int n4 = vec ? n / 4 : 0;
#pragma unroll
            for (int u = 0; u < QU; ++u) {
                const int q = tid + u * NT;
                const int qc = q < n4 ? q : (n4 > 0 ? n4 - 1 : 0);
                v[u][0] = n4 > 0 ? reinterpret_cast<const float4*>(G)[qc] : make_float4(0.0f, 0.0f, 0.0f, 0.0f);
            }
        }
    }
    __device__ inline void store(float* gs, const float* __restrict__ G, int nidx, int B)
    {
        const int tid = threadIdx.x;
        if (!vec) {
            // unaligned or ragged source: element by element
            for (int q = tid; q < nidx * NB; q += NT) {
                const int i = q / NB;
                const int b = q - i * NB;
                gs[q] = RM ? (b < B ? G[(int64_t)b * nidx + i] : 0.0f) : G[q];
            }
            return;
        }
        if constexpr (RM) {
            const int n4 = nidx / 4;
#pragma unroll
            for (int u = 0; u < QU; ++u) {
                const int q = tid + u * NT;
                if (q >= n4) break;
                float4 w[NB];
#pragma unroll
                for (int b = 0; b < NB; ++b) w[b] = b < B ? v[u][b] : make_float4(0.0f, 0.0f, 0.0f, 0.0f);
                float4* d = reinterpret_cast<float4*>(gs + q * 4 * NB);
                if constexpr (NB == 4) {
                    d[0] = make_float4(w[0].x, w[1].x, w[2].x, w[3].x);
                    d[1] = make_float4(w[0].y, w[1].y, w[2].y, w[3].y);
                    d[2] = make_float4(w[0].z, w[1].z, w[2].z, w[3].z);
                    d[3] = make_float4(w[0].w, w[1].w, w[2].w, w[3].w);
                } else if constexpr (NB == 2) {
                    d[0] = make_float4(w[0].x, w[1].x, w[0].y, w[1].y);
                    d[1] = make_float4(w[0].z, w[1].z, w[0].w, w[1].w);
                } else {
                    d[0] = w[0];
                }
            }
        } else {
            const int n4 = nidx * NB / 4;
#pragma unroll
            for (int u = 0; u < QU; ++u) {
                const int q = tid + u * NT;
                if (q >= n4) break;
                reinterpret_cast<float4*>(gs)[q] = v[u][0];
            }
        }
    }
};

// One role of the streamed kernel on workgroup vb of the nwg that take it.
// V16: the values come from their bf16 copy (forward only).
template <int NB, int D, bool DW, bool SPMM, bool RM, bool VAL, bool I16, bool V16 = false>
__device__ __forceinline__ void stream_role(const RoleArgs& A, int bp, int B, int vb, int nwg)
{
    static_assert(NB == 1 || NB == 2 || NB == 4, "one to four columns per lane");
    extern __shared__ __align__(16) float gs_dyn[];
    const int lane = threadIdx.x & (kWave - 1);
    const int wv = uni((int)(threadIdx.x / kWave));
    const int nidx = A.nidx;
    const int nkeys = A.nkeys;
    constexpr bool LV = SPMM || VAL;

    // wavefront gw of the grid takes an even share of the keys (workgroups of
    // one XCD adjacent shares)
    StreamCursor cur;
    cur.ptr = A.ptr;
    cur.nkeys = nkeys;
    {
        const int64_t nw = (int64_t)nwg * kLdsKeyWaves;
        const int64_t gw = (int64_t)vb * kLdsKeyWaves + wv;
        cur.start((int32_t)(nkeys * gw / nw), (int32_t)(nkeys * (gw + 1) / nw), lane);
    }

    // the ring: D blocks in flight (indices, values, the key's dW operand and
    // the MSE target of the lane's column), refilled as each is consumed
    StreamDesc d[D];
    int4 bi[D];
    float4 bv[D];
    float hb[D][NB];
    float tq[D];
    // the column whose output this lane would store at a key's end (see the key-end reduction)
    const int tcol0 = NB == 4 ? (lane >> 4) : (NB == 2 ? (lane >> 5) : 0);
    const int tcol = tcol0 < B ? tcol0 : B - 1;
    auto issue = [&](int q) {
        cur.next(d[q], lane);
        const int32_t o = d[q].base + 4 * lane;
        if constexpr (I16) {
            // four 16-bit indices in 8 bytes: the index stream at half the bytes
            const uint2 u = *reinterpret_cast<const uint2*>(A.idx16 + o);
            bi[q] = make_int4((int)(u.x & 0xffffu), (int)(u.x >> 16), (int)(u.y & 0xffffu), (int)(u.y >> 16));
        } else {
            bi[q] = *reinterpret_cast<const int4*>(A.idx + o);
        }
        if constexpr (V16) {
            // four bf16 values in 8 bytes, widened exactly
            const uint2 u = *reinterpret_cast<const uint2*>(A.vals16 + o);
            bv[q] = make_float4(__uint_as_float(u.x << 16), __uint_as_float(u.x & 0xFFFF0000u),
                                __uint_as_float(u.y << 16), __uint_as_float(u.y & 0xFFFF0000u));
        } else if constexpr (LV) {
            bv[q] = *reinterpret_cast<const float4*>(A.vals + o);
        }
        if constexpr (DW) load_h<NB, RM>(A.H, d[q].r, bp, 0, B, nkeys, hb[q]);
        if constexpr (SPMM) tq[q] = A.tgt[(int64_t)tcol * nkeys + d[q].r];
    };

    // stage the operand (and the zero row after it): every load of this
    // thread's share is issued at once, then the ring's first blocks, then the
    // staged values are stored -- so the staging and the first blocks share one
    // memory latency
    StreamStage<NB, RM> st;
    st.load(A.G, nidx, B);
#pragma unroll
    for (int q = 0; q < D; ++q) issue(q);
    st.store(gs_dyn, A.G, nidx, B);
    if (threadIdx.x < NB) gs_dyn[nidx * NB + threadIdx.x] = 0.0f;
    __syncthreads();

    float acc[NB];
#pragma unroll
    for (int n = 0; n < NB; ++n) acc[n] = 0.0f;
    for (;;) {
#pragma unroll
        for (int q = 0; q < D; ++q) {
            const StreamDesc dq = d[q];
            const int32_t k0 = dq.base + 4 * lane;
            const int32_t ii[4] = {bi[q].x, bi[q].y, bi[q].z, bi[q].w};
            const float vv[4] = {bv[q].x, bv[q].y, bv[q].z, bv[q].w};
            bool in[4];
            float y[4][NB];
#pragma unroll
            for (int t = 0; t < 4; ++t) {
                in[t] = k0 + t >= dq.lo && k0 + t < dq.hi;
                lds_row<NB>(gs_dyn, in[t] ? ii[t] : nidx, y[t]);
            }
            if constexpr (SPMM) {
#pragma unroll
                for (int t = 0; t < 4; ++t) {
                    const float v = in[t] ? vv[t] : 0.0f;
#pragma unroll
                    for (int n = 0; n < NB; ++n) acc[n] = fmaf(v, y[t][n], acc[n]);
                }
            }
            if constexpr (DW) {
                float g[4];
#pragma unroll
                for (int t = 0; t < 4; ++t) {
                    float a = 0.0f;
#pragma unroll
                    for (int n = 0; n < NB; ++n) a = fmaf(y[t][n], hb[q][n], a);
                    g[t] = a;
                }
                float* __restrict__ dwo = A.dwo;
                float* __restrict__ apply = A.apply;
                if (in[0] && in[3]) {
                    if (dwo) *reinterpret_cast<float4*>(dwo + k0) = make_float4(g[0], g[1], g[2], g[3]);
                    if (apply)
                        *reinterpret_cast<float4*>(apply + k0) =
                            make_float4(sgd_value(vv[0], g[0], A.lr), sgd_value(vv[1], g[1], A.lr),
                                        sgd_value(vv[2], g[2], A.lr), sgd_value(vv[3], g[3], A.lr));
                } else {
#pragma unroll
                    for (int t = 0; t < 4; ++t) {
                        if (in[t]) {
                            if (dwo) dwo[k0 + t] = g[t];
                            if (apply) apply[k0 + t] = sgd_value(vv[t], g[t], A.lr);
                        }
                    }
                }
            }
            if constexpr (SPMM) {
                if (dq.flags & 2) {
                    // the key's sums over the wavefront (fixed trees): lane sl ends
                    // with the total of column sc and stores it
                    float sv;
                    int sc, sl;
                    if constexpr (NB == 4) {
                        // halves exchanged over lane bits 5 and 4, then sums over bits 3-0:
                        // lane 16 c holds column c
                        sv = group_reduce<1, 4>(acc, lane);
                        sc = lane >> 4;
                        sl = sc << 4;
                    } else if constexpr (NB == 2) {
                        // halves exchanged over lane bit 5, then sums over bits 4-0:
                        // lane 32 c holds column c
                        xlevel<5, 2, 2>(acc, lane);
                        sv = acc[0];
                        sv += __shfl_xor(sv, 16, kWave);
                        sv += lane_xor<8>(sv);
                        sv += lane_xor<4>(sv);
                        sv += lane_xor<2>(sv);
                        sv += lane_xor<1>(sv);
                        sc = lane >> 5;
                        sl = sc << 5;
                    } else {
                        sv = wave_sum(acc[0]);
                        sc = 0;
                        sl = 0;
                    }
                    if (lane == sl && sc < B) {
                        const int64_t o = (int64_t)sc * nkeys + dq.r;
                        if (A.act == kActGelu) sv = gelu_value(sv);
                        A.out[o] = sv;
                        if (A.dyo) A.dyo[o] = A.mse_scale * (sv - tq[q]);
                    }
#pragma unroll
                    for (int n = 0; n < NB; ++n) acc[n] = 0.0f;
                }
            }
            issue(q);
        }
        if (!d[0].valid()) break;
    }
}

// workgroup index with the workgroups of one XCD adjacent (the grid is a multiple of kXcd)
__device__ inline int xcd_major_block()
{
    const int nwg = (int)gridDim.x;
    const int bid = (int)blockIdx.x;
    return (bid % kXcd) * (nwg / kXcd) + bid / kXcd;
}

template <int NB, int D, bool DW, bool SPMM, bool RM, bool VAL, bool I16, bool V16 = false>
__global__ void __launch_bounds__(kLdsKeyWaves * kWave) stream_lds_kernel(RoleArgs A, int bp, int B)
{
    stream_role<NB, D, DW, SPMM, RM, VAL, I16, V16>(A, bp, B, xcd_major_block(), (int)gridDim.x);
}

// The two passes of a backward with dX and dW in one launch: workgroups
// [0, g0) run the column pass (dX, and dW in column order or the column-ordered
// values stepped), the rest the row pass (dW in canonical order, optionally the
// canonical values stepped).  The passes are independent, so they overlap
// instead of paying two launches and two ramps; the split follows their bytes.
template <int NB, int D, bool RM, bool I16, bool VALR>
__global__ void __launch_bounds__(kLdsKeyWaves * kWave) stream_bwd_kernel(RoleArgs Ac, RoleArgs Ar, int g0, int bp,
                                                                          int B)
{
    const int vb = xcd_major_block();
    if (vb < g0) stream_role<NB, D, true, true, RM, true, I16>(Ac, bp, B, vb, g0);
    else stream_role<NB, D, true, false, RM, VALR, I16>(Ar, bp, B, vb - g0, (int)gridDim.x - g0);
}

// out[b, r] = sum over slices s = 0, 1, ... of part[s][r][b], in that order
template <int BTILE>
constexpr int kSplitReduceKeys = 1024 / BTILE;   // keys per workgroup of split_reduce_kernel

// With dyo: dyo = scale * (out - tgt) beside out, and with dyt also the
// feature-major copy dyt[r * BTILE + b] (zero for b >= B).
struct MseOut {
    const float* tgt;
    float* dyo;
    float* dyt;
    float scale;
};

template <int BTILE>
__global__ void __launch_bounds__(256) split_reduce_kernel(const float* __restrict__ part, int S, int nkeys, int B,
                                                           float* __restrict__ out, MseOut mse)
{
    constexpr int Q = BTILE / 4;
    constexpr int KPB = kSplitReduceKeys<BTILE>;   // one float4 of the tile per thread
    constexpr int NOUT = KPB * BTILE / 256;        // output elements per thread
    __shared__ float t[KPB][BTILE + 1];
    const int r0 = (int)blockIdx.x * KPB;
    const int64_t sstride = (int64_t)nkeys * Q;
    // batch tile blockIdx.y: its partial sums, and its rows of the batch-major
    // arrays (outputs, targets, gradient)
    part += (int64_t)blockIdx.y * S * nkeys * BTILE;
    out += (int64_t)blockIdx.y * BTILE * nkeys;
    if (mse.dyo) {
        mse.tgt += (int64_t)blockIdx.y * BTILE * nkeys;
        mse.dyo += (int64_t)blockIdx.y * BTILE * nkeys;
    }
    B -= (int)blockIdx.y * BTILE;
    // the targets of this thread's outputs, loaded first so they arrive with the
    // partial sums (clamped, unconditional loads: without a gradient they come
    // from part, which is longer than any [B][nkeys] array)
    float tg[NOUT];
    {
        const float* __restrict__ src = mse.dyo ? mse.tgt : part;
#pragma unroll
        for (int i = 0; i < NOUT; ++i) {
            const int e = (int)threadIdx.x + 256 * i;
            const int b = e / KPB;
            const int r = r0 + (e - b * KPB);
            tg[i] = src[(int64_t)(b < B ? b : B - 1) * nkeys + (r < nkeys ? r : nkeys - 1)];
        }
    }
    for (int e = threadIdx.x; e < KPB * Q; e += 256) {
        const int kk = e / Q;
        const int c4 = e - kk * Q;
        const int r = r0 + kk;
        float4 a = make_float4(0.0f, 0.0f, 0.0f, 0.0f);
        if (r < nkeys) {
            const float4* __restrict__ pp = reinterpret_cast<const float4*>(part) + (int64_t)r * Q + c4;
#pragma unroll 8
            for (int s = 0; s < S; ++s) {
                const float4 v = pp[s * sstride];
                a.x += v.x;
                a.y += v.y;
                a.z += v.z;
                a.w += v.w;
            }
        }
        t[kk][c4 * 4 + 0] = a.x;
        t[kk][c4 * 4 + 1] = a.y;
        t[kk][c4 * 4 + 2] = a.z;
        t[kk][c4 * 4 + 3] = a.w;
    }
    __syncthreads();
#pragma unroll
    for (int i = 0; i < NOUT; ++i) {
        const int e = (int)threadIdx.x + 256 * i;
        const int b = e / KPB;
        const int kk = e - b * KPB;
        const int r = r0 + kk;
        if (b < B && r < nkeys) {
            const int64_t o = (int64_t)b * nkeys + r;
            out[o] = t[kk][b];
            if (mse.dyo) {
                const float d = mse.scale * (t[kk][b] - tg[i]);
                mse.dyo[o] = d;
                t[kk][b] = d;   // only this thread reads (kk, b)
            }
        }
    }
    if (mse.dyo && mse.dyt) {
        __syncthreads();
        for (int e = threadIdx.x; e < KPB * Q; e += 256) {
            const int kk = e / Q;
            const int b = (e - kk * Q) * 4;
            const int r = r0 + kk;
            if (r < nkeys)
                *reinterpret_cast<float4*>(mse.dyt + (int64_t)r * BTILE * gridDim.y + blockIdx.y * BTILE + b) =
                    make_float4(b < B ? t[kk][b] : 0.0f, b + 1 < B ? t[kk][b + 1] : 0.0f,
                                b + 2 < B ? t[kk][b + 2] : 0.0f, b + 3 < B ? t[kk][b + 3] : 0.0f);
        }
    }
}

// The slice tables of one view for up to kTileWidths slice counts in one
// pass over its index: a wavefront per key reads the key's ascending indices
// once; an entry whose slice passes its predecessor's is the first entry of
// every slice in between (tab[s * nkeys + key]), slices up to the first entry's
// start at the key's first entry and slices past the last entry at its end.
struct TabSet {
    int32_t S[kTileWidths];
    int32_t* tab[kTileWidths];   // null: not built
    double inv_nidx;             // 1 / nidx
};

// the slice s with split_start(s) <= i < split_start(s + 1), i.e.
// floor(((i + 1) S - 1) / nidx); the numerator is an integer below 2^38 and
// the exact quotient's distance from the next integer is at least 1 / nidx,
// far above the rounding error of the reciprocal product, so the floor is exact
__device__ inline int32_t slice_of(int32_t i, int32_t S, double inv_nidx)
{
    return (int32_t)floor(((double)(i + 1) * (double)S - 1.0) * inv_nidx);
}

__global__ void __launch_bounds__(256) split_tables_kernel(const int32_t* __restrict__ ptr,
                                                           const int32_t* __restrict__ idx, int32_t nkeys,
                                                           int32_t nidx, TabSet ts)
{
    const int lane = threadIdx.x & (kWave - 1);
    const int32_t r = (int32_t)blockIdx.x * (256 / kWave) + (int32_t)(threadIdx.x / kWave);
    if (r >= nkeys) return;
    const int32_t p0 = ptr[r], p1 = ptr[r + 1];
    int32_t carry[kTileWidths];   // slice of the entry before this step's first
#pragma unroll
    for (int w = 0; w < kTileWidths; ++w) carry[w] = -1;
    for (int32_t base = p0; base < p1; base += kWave) {
        const int32_t k = base + lane;
        const int32_t i = idx[k < p1 ? k : p1 - 1];
#pragma unroll
        for (int w = 0; w < kTileWidths; ++w) {
            if (!ts.tab[w]) continue;
            const int32_t S = ts.S[w];
            const int32_t t = slice_of(i, S, ts.inv_nidx);
            const int32_t up = __shfl_up(t, 1, kWave);
            const int32_t tp = lane == 0 ? carry[w] : up;
            carry[w] = __shfl(t, kWave - 1, kWave);
            if (k < p1)
                for (int32_t sl = tp + 1; sl <= t; ++sl) ts.tab[w][(int64_t)sl * nkeys + r] = k;
        }
    }
#pragma unroll
    for (int w = 0; w < kTileWidths; ++w) {
        if (!ts.tab[w]) continue;
        const int32_t S = ts.S[w];
        const int32_t tl = p1 > p0 ? slice_of(idx[p1 - 1], S, ts.inv_nidx) : -1;
        for (int32_t sl = tl + 1 + lane; sl <= S; sl += kWave) ts.tab[w][(int64_t)sl * nkeys + r] = p1;
    }
}

// dW in canonical order from dW in transposed order: dw[k] = dwt[iperm[k]].
// XCD x owns one contiguous eighth of the canonical slots (one eighth of the
// rows); its workgroups sweep that range together, workgroup w taking chunks
// w, w + nw, ..., so at any moment the XCD works on a narrow window of rows and
// the column-order lines those rows reach stay in its L2 until all their
// entries have been read.
__global__ void __launch_bounds__(kBlock) permute_dw_kernel(const int32_t* __restrict__ iperm,
                                                            const float* __restrict__ dwt, int64_t nnz,
                                                            int64_t per_xcd, float* __restrict__ dw)
{
    const int x = (int)blockIdx.x % kXcd;
    const int64_t w = blockIdx.x / kXcd, nw = gridDim.x / kXcd;
    const int64_t k0 = (int64_t)x * per_xcd;
    const int64_t k1 = k0 + per_xcd < nnz ? k0 + per_xcd : nnz;
    for (int64_t k = k0 + w * kBlock + threadIdx.x; k < k1; k += 2 * nw * kBlock) {
        const int64_t k2 = k + nw * kBlock;
        const int32_t j0 = iperm[k];
        const int32_t j1 = k2 < k1 ? iperm[k2] : j0;
        const float v0 = dwt[j0], v1 = dwt[j1];
        dw[k] = v0;
        if (k2 < k1) dw[k2] = v1;
    }
}

// dW in canonical order from the column order, one tile of the matrix per
// workgroup: the entries whose rows lie in slice a of the column view's split
// table and whose columns lie in slice b of the row view's.  Inside a tile each
// column's entries are one run of the column order and each row's one run of
// the canonical order, so the tile's column-order dW is copied into LDS run by
// run and the canonical runs are written from there (an entry's LDS place is
// its column's offset plus its rank in the column, from iperm): every global
// access is a run about a cache line long instead of a scattered word.  A
// half wavefront takes a run, kPermU runs at a time so their loads overlap
// (the kernel waits on memory, not on issue).  A tile larger than the buffer
// gathers directly.
constexpr int kPermThreads = 1024;
constexpr int kPermWaves = kPermThreads / kWave;
constexpr int kPermU = 10;   // runs per half wavefront in flight

struct PermArgs {
    const int32_t* ttab;   // column view: column c's run in row slice a is [ttab[a*ts + c], ttab[(a+1)*ts + c])
    int64_t ts;
    const int32_t* ftab;   // row view: row r's run in column slice b is [ftab[b*fs + r], ftab[(b+1)*fs + r])
    int64_t fs;
    int32_t SA, SB, M, K;
    int32_t cap;             // entries the LDS buffer holds
    int32_t ncmax, nrmax;    // most columns / rows of a tile
    const int32_t* iperm;
    const int32_t* cols;
    const float* dwt;
    float* dw;
};

__global__ void __launch_bounds__(kPermThreads) permute_tiles_kernel(PermArgs P)
{
    extern __shared__ __align__(16) float pt_dyn[];
    __shared__ int32_t wsum[kPermWaves];
    float* ent = pt_dyn;
    int32_t* cbeg = reinterpret_cast<int32_t*>(pt_dyn + P.cap);   // [ncmax] a column run's first slot
    int32_t* coff = cbeg + P.ncmax;                                // [ncmax + 1] its place in ent
    int32_t* rbeg = coff + P.ncmax + 1;                            // [nrmax] a row run's bounds
    int32_t* rend = rbeg + P.nrmax;
    const int a = (int)blockIdx.x / P.SB, b = (int)blockIdx.x % P.SB;
    const int32_t r0 = split_start(a, P.SA, P.M), nr = split_start(a + 1, P.SA, P.M) - r0;
    const int32_t c0 = split_start(b, P.SB, P.K), nc = split_start(b + 1, P.SB, P.K) - c0;
    const int tid = (int)threadIdx.x, lane = tid & (kWave - 1), wv = tid / kWave;

    // column runs and their exclusive prefix (each thread a few consecutive columns)
    const int per = (nc + kPermThreads - 1) / kPermThreads;
    int32_t loc = 0;
    for (int i = 0; i < per; ++i) {
        const int ci = tid * per + i;
        if (ci < nc) {
            const int32_t s0 = P.ttab[(int64_t)a * P.ts + c0 + ci];
            const int32_t s1 = P.ttab[(int64_t)(a + 1) * P.ts + c0 + ci];
            cbeg[ci] = s0;
            coff[ci] = s1 - s0;
            loc += s1 - s0;
        }
    }
    int32_t inc = loc;
#pragma unroll
    for (int o = 1; o < kWave; o <<= 1) {
        const int32_t t = __shfl_up(inc, o, kWave);
        if (lane >= o) inc += t;
    }
    if (lane == kWave - 1) wsum[wv] = inc;
    for (int ri = tid; ri < nr; ri += kPermThreads) {
        rbeg[ri] = P.ftab[(int64_t)b * P.fs + r0 + ri];
        rend[ri] = P.ftab[(int64_t)(b + 1) * P.fs + r0 + ri];
    }
    __syncthreads();
    int32_t run = inc - loc;
    for (int w = 0; w < wv; ++w) run += wsum[w];
    for (int i = 0; i < per; ++i) {
        const int ci = tid * per + i;
        if (ci < nc) {
            const int32_t len = coff[ci];
            coff[ci] = run;
            run += len;
        }
    }
    if (tid == kPermThreads - 1) coff[nc] = run;
    __syncthreads();
    const int32_t E = coff[nc];
    if (E > P.cap) {   // uniform: gather the tile's row runs directly
        for (int ri = wv; ri < nr; ri += kPermWaves) {
            const int32_t k1 = rend[ri];
            for (int32_t k = rbeg[ri] + lane; k < k1; k += kWave) P.dw[k] = P.dwt[P.iperm[k]];
        }
        return;
    }
    const int half = lane >> 5, hl = lane & 31;
    // column runs into LDS
    for (int c = wv * 2 * kPermU; c < nc; c += kPermWaves * 2 * kPermU) {
        int32_t sb[kPermU], so[kPermU], sl[kPermU], mx = 0;
#pragma unroll
        for (int u = 0; u < kPermU; ++u) {
            const int ci = c + 2 * u + half;
            const bool ok = ci < nc;
            sb[u] = ok ? cbeg[ci] : 0;
            so[u] = ok ? coff[ci] : 0;
            sl[u] = ok ? coff[ci + 1] - coff[ci] : 0;
            mx = max(mx, sl[u]);
        }
        for (int t = hl; t < mx; t += 32) {
            float v[kPermU];
#pragma unroll
            for (int u = 0; u < kPermU; ++u) v[u] = P.dwt[sb[u] + min(t, max(sl[u] - 1, 0))];
#pragma unroll
            for (int u = 0; u < kPermU; ++u)
                if (t < sl[u]) ent[so[u] + t] = v[u];
        }
    }
    __syncthreads();
    // canonical row runs from LDS
    for (int r = wv * 2 * kPermU; r < nr; r += kPermWaves * 2 * kPermU) {
        int32_t kb[kPermU], kl[kPermU], mx = 0;
#pragma unroll
        for (int u = 0; u < kPermU; ++u) {
            const int ri = r + 2 * u + half;
            const bool ok = ri < nr;
            kb[u] = ok ? rbeg[ri] : 0;
            kl[u] = ok ? rend[ri] - rbeg[ri] : 0;
            mx = max(mx, kl[u]);
        }
        for (int t = hl; t < mx; t += 32) {
            int32_t j[kPermU], c[kPermU];
#pragma unroll
            for (int u = 0; u < kPermU; ++u) {
                const int32_t k = kb[u] + min(t, max(kl[u] - 1, 0));
                j[u] = P.iperm[k];
                c[u] = P.cols[k];
            }
#pragma unroll
            for (int u = 0; u < kPermU; ++u) {
                if (t < kl[u]) {
                    const int ci = c[u] - c0;
                    P.dw[kb[u] + t] = ent[coff[ci] + (j[u] - cbeg[ci])];
                }
            }
        }
    }
}

// dW[k] = sum_b dyt[r_k, b] * xt[c_k, b] over several batch tiles (batches
// wider than one tile); group g of a wave step takes U consecutive slots and
// its BT lanes are reduced by a butterfly.
template <int BT, int NB, int U>
__global__ void __launch_bounds__(kBlock) sddmm_tiles_kernel(const int32_t* __restrict__ rows,
                                                             const int32_t* __restrict__ cols, int64_t nnz,
                                                             const float* __restrict__ xt,
                                                             const float* __restrict__ dyt, int bp, int ntiles,
                                                             float* __restrict__ dW, int64_t nsteps)
{
    constexpr int G = kWave / BT;
    constexpr int STEP = G * U;
    const int lane = threadIdx.x & (kWave - 1);
    const int g = lane / BT;
    const int bl = lane - g * BT;
    const int64_t nwaves = (int64_t)gridDim.x * kWavesPerBlock;
    for (int64_t st = (int64_t)blockIdx.x * kWavesPerBlock + threadIdx.x / kWave; st < nsteps; st += nwaves) {
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
#pragma unroll
        for (int u = 0; u < U; ++u)
            if ((u % BT) == bl && my + u < nnz) dW[my + u] = acc[u];
    }
}

RoleArgs role_for(const View& v, const float* G, const float* H, float* out, float* dwo, int wpb, int64_t cap)
{
    RoleArgs a;
    a.cap = cap;
    a.idx = v.idx;
    a.idx16 = v.idx16;
    a.vals16 = nullptr;
    a.act = kActNone;
    a.vals = v.vals;
    a.ptr = v.ptr;
    a.desc = v.desc;
    a.empty_keys = v.empty_keys;
    a.n_empty = v.n_empty;
    a.G = G;
    a.H = H;
    a.out = out;
    a.dwo = dwo;
    a.apply = nullptr;
    a.lr = 0.0f;
    a.tgt = nullptr;
    a.dyo = nullptr;
    a.dyto = nullptr;
    a.mse_scale = 0.0f;
    a.nchunks = v.nchunks;
    a.nkeys = v.nkeys;
    a.nidx = v.nidx;
    a.nblocks = (v.nchunks + wpb - 1) / wpb;
    a.per_xcd = (a.nblocks + kXcd - 1) / kXcd;
    return a;
}

constexpr int kXldsBytes = 64 * 1024;   // largest operand staged in LDS
constexpr int kXldsWaves = 8;

template <int BT, int NB, int P, bool DW, int WPB, bool XLDS>
snack_status launch_seg(const RoleArgs& a, const RoleArgs* b, int ntiles, int bp, int B, hipStream_t s)
{
    const int grid_a = a.per_xcd * kXcd;
    const int grid_b = b ? b->per_xcd * kXcd : 0;
    RoleArgs bb = b ? *b : a;
    dim3 grid((unsigned)(grid_a + grid_b), (unsigned)ntiles);
    size_t dyn = 0;
    if (XLDS) {
        const size_t na = (size_t)a.nidx * bp * 4, nb = b ? (size_t)b->nidx * bp * 4 : 0;
        dyn = na > nb ? na : nb;
    }
    hipLaunchKernelGGL((seg_kernel<BT, NB, P, DW, WPB, XLDS>), grid, dim3(WPB * kWave), dyn, s, a, bb, grid_a, bp, B);
    SNACK_HIP(hipGetLastError());
    return SNACK_OK;
}

// operands small enough for LDS are staged there (B = 1 at up to 16K features)
inline bool use_xlds(const BatchPlan& p, int nidx_max)
{
    return p.btile == 1 && (size_t)nidx_max * p.bp * 4 <= (size_t)kXldsBytes;
}

template <bool DW>
snack_status dispatch_seg(const BatchPlan& p, int64_t cap, const View& va, const float* Ga, const float* Ha,
                          float* outa, float* dwa, const View* vbv, const float* Gb, const float* Hb, float* dwb,
                          int B, hipStream_t s)
{
    const int nmax = vbv && vbv->nidx > va.nidx ? vbv->nidx : va.nidx;
    if (use_xlds(p, nmax)) {
        const RoleArgs a = role_for(va, Ga, Ha, outa, dwa, kXldsWaves, cap);
        RoleArgs b;
        if (vbv) b = role_for(*vbv, Gb, Hb, nullptr, dwb, kXldsWaves, cap);
        return launch_seg<1, 1, 2, DW, kXldsWaves, true>(a, vbv ? &b : nullptr, p.ntiles, p.bp, B, s);
    }
    const RoleArgs a = role_for(va, Ga, Ha, outa, dwa, kWavesPerBlock, cap);
    RoleArgs b;
    if (vbv) b = role_for(*vbv, Gb, Hb, nullptr, dwb, kWavesPerBlock, cap);
    const RoleArgs* pb = vbv ? &b : nullptr;
    switch (p.btile) {
    case 1: return launch_seg<1, 1, 2, DW, kWavesPerBlock, false>(a, pb, p.ntiles, p.bp, B, s);
    case 2: return launch_seg<1, 2, 2, DW, kWavesPerBlock, false>(a, pb, p.ntiles, p.bp, B, s);
    case 4: return launch_seg<1, 4, 2, DW, kWavesPerBlock, false>(a, pb, p.ntiles, p.bp, B, s);
    case 8: return launch_seg<1, 8, 1, DW, kWavesPerBlock, false>(a, pb, p.ntiles, p.bp, B, s);
    case 16: return launch_seg<2, 8, 1, DW, kWavesPerBlock, false>(a, pb, p.ntiles, p.bp, B, s);
    case 32: return launch_seg<4, 8, 1, DW, kWavesPerBlock, false>(a, pb, p.ntiles, p.bp, B, s);
    case 64: return launch_seg<8, 8, 1, DW, kWavesPerBlock, false>(a, pb, p.ntiles, p.bp, B, s);
    default: return SNACK_ERR_INVALID_ARG;
    }
}

// key-major kernels: worth it where gathers dominate (wide batch tiles) and
// keys are long enough to keep every group busy
// widest batch tile that recomputes dW over the row view instead of permuting
// the column-order dW; up to here every kernel pair that can meet gives each
// lane the same batch columns, so the two dW orders agree bit for bit
constexpr int kKeyedRecomputeMax = 32;

inline bool use_keyed(const View& v, int64_t nnz, const BatchPlan& p)
{
    return p.btile >= 1 && v.nkeys > 0 && nnz / v.nkeys >= 128;
}

// LDS of the streamed kernel: the operand and one zero row
inline size_t stream_lds_bytes(const View& v, const BatchPlan& p)
{
    return ((size_t)v.nidx + 1) * p.bp * sizeof(float);
}

// the streamed kernel with the whole gathered operand in LDS applies: its
// blocks never span two keys, so keys down to 16 entries on average still pay
// (a block's loads then cover neighbouring keys, which the next block re-reads
// from the L2)
constexpr int64_t kStreamMinKey = 16;
inline bool keyed_lds(const snack_layer* L, const View& v, const BatchPlan& p)
{
    return p.btile <= 4 && p.ntiles == 1 && L->cus > 0 && v.nchunks > 0 && v.nkeys > 0 &&
           L->nnz / v.nkeys >= kStreamMinKey && stream_lds_bytes(v, p) <= (size_t)L->lds_bytes;
}

// blocks in flight per wavefront of the streamed kernel (registers allow more
// at narrower tiles)
#ifndef SNACK_STREAM_D1
#define SNACK_STREAM_D1 8
#endif
#ifndef SNACK_STREAM_D2
#define SNACK_STREAM_D2 6
#endif
#ifndef SNACK_STREAM_D4
#define SNACK_STREAM_D4 4
#endif
template <int NB>
constexpr int kStreamDepthFor = NB == 4 ? SNACK_STREAM_D4 : (NB == 2 ? SNACK_STREAM_D2 : SNACK_STREAM_D1);

// rm: G and H are batch-major [B][n] (the caller's arrays); only the LDS
// kernel takes them, transposing G while it stages it
// VAL: load the entries' values in a dW-only pass (needed for `apply`)
// mse: the MSE gradient written beside the output by the key stores (batch-major only)
template <bool DW, bool SPMM = true, bool VAL = false>
snack_status launch_keyed(const BatchPlan& p, const snack_layer* L, const View& v, const float* G, const float* H,
                          float* out, float* dwo, int B, hipStream_t s, bool rm = false, float* apply = nullptr,
                          float lr = 0.0f, MseFuse* mse = nullptr)
{
    constexpr bool LV = SPMM || VAL;
    if (apply && !LV) return SNACK_ERR_INVALID_ARG;   // the step needs the values
    if (mse && !SPMM) return SNACK_ERR_INVALID_ARG;
    RoleArgs a = role_for(v, G, H, out, dwo, kWavesPerBlock, L->cap);
    a.apply = apply;
    a.lr = lr;
    a.tgt = out;   // the key stores read targets unconditionally: any valid [B][nkeys] array
    if (mse) {
        a.tgt = mse->T;
        a.dyo = mse->dY;
        a.mse_scale = mse->scale;
        mse->done = true;
    }
    const size_t lds = stream_lds_bytes(v, p);
    if (p.btile <= 4 && p.ntiles == 1 && lds <= (size_t)L->lds_bytes && L->cus > 0 && v.nchunks > 0) {
        // operand resident in LDS: persistent workgroups, as many per CU as stay
        // resident together (at most two), each wavefront an even share of the keys
        const dim3 block(kLdsKeyWaves * kWave);
        auto go = [&](auto kern) {
            int occ = 1;
            if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&occ, kern, (int)block.x, lds) != hipSuccess || occ < 1)
                occ = 1;
            int nwg = L->cus * (occ > 2 ? 2 : occ);
            const int want = (v.nkeys + kLdsKeyWaves - 1) / kLdsKeyWaves;   // no workgroup without keys
            if (nwg > want) nwg = want;
            nwg = (nwg + kXcd - 1) / kXcd * kXcd;
            hipLaunchKernelGGL(kern, dim3((unsigned)nwg), block, lds, s, a, p.bp, B);
        };
        auto pick = [&](auto rmc, auto i16c) {
            constexpr bool R = decltype(rmc)::value, I = decltype(i16c)::value;
            switch (p.btile) {
            case 1: go(stream_lds_kernel<1, kStreamDepthFor<1>, DW, SPMM, R, LV, I>); return true;
            case 2: go(stream_lds_kernel<2, kStreamDepthFor<2>, DW, SPMM, R, LV, I>); return true;
            case 4: go(stream_lds_kernel<4, kStreamDepthFor<4>, DW, SPMM, R, LV, I>); return true;
            default: return false;
            }
        };
        using T = std::true_type;
        using F = std::false_type;
        const bool i16 = v.idx16 != nullptr;
        const bool ok = rm ? (i16 ? pick(T{}, T{}) : pick(T{}, F{})) : (i16 ? pick(F{}, T{}) : pick(F{}, F{}));
        if (!ok) return SNACK_ERR_INVALID_ARG;
        SNACK_HIP(hipGetLastError());
        return SNACK_OK;
    }
    if (rm) return SNACK_ERR_INVALID_ARG;   // callers check spmm_batch_major first
    dim3 grid((unsigned)(a.per_xcd * kXcd), (unsigned)p.ntiles);
    switch (p.btile) {
    case 1: hipLaunchKernelGGL((key_kernel<1, 1, 4, DW, SPMM, LV>), grid, dim3(kBlock), 0, s, a, p.bp, B); break;
    case 2: hipLaunchKernelGGL((key_kernel<1, 2, 4, DW, SPMM, LV>), grid, dim3(kBlock), 0, s, a, p.bp, B); break;
    case 4: hipLaunchKernelGGL((key_kernel<1, 4, 4, DW, SPMM, LV>), grid, dim3(kBlock), 0, s, a, p.bp, B); break;
    case 8: hipLaunchKernelGGL((key_kernel<2, 4, 4, DW, SPMM, LV>), grid, dim3(kBlock), 0, s, a, p.bp, B); break;
    case 16: hipLaunchKernelGGL((key_kernel<4, 4, 4, DW, SPMM, LV>), grid, dim3(kBlock), 0, s, a, p.bp, B); break;
    case 32: hipLaunchKernelGGL((key_kernel<4, 8, 4, DW, SPMM, LV>), grid, dim3(kBlock), 0, s, a, p.bp, B); break;
    case 64: hipLaunchKernelGGL((key_kernel<8, 8, 4, DW, SPMM, LV>), grid, dim3(kBlock), 0, s, a, p.bp, B); break;
    default: return SNACK_ERR_INVALID_ARG;
    }
    SNACK_HIP(hipGetLastError());
    return SNACK_OK;
}

// dX and dW at batch tiles 1-4 with both operands in LDS: the column pass over
// the transposed view (dX; dW in column order into dwo_t unless null; with
// apply_t its values stepped in place) and the row pass over the canonical view
// (dW; with apply its values stepped) in one launch of the two-role kernel.
snack_status launch_stream_bwd(const BatchPlan& p, const snack_layer* L, const float* dyt, const float* xt, float* dX,
                               float* dwo_t, float* apply_t, float* dW, float* apply, float lr, int B, hipStream_t s,
                               bool rm)
{
    if (!keyed_lds(L, L->tr, p) || !keyed_lds(L, L->fwd, p)) return SNACK_ERR_INVALID_ARG;
    RoleArgs ac = role_for(L->tr, dyt, xt, dX, dwo_t, kWavesPerBlock, L->cap);
    ac.apply = apply_t;
    ac.lr = lr;
    ac.tgt = dX;   // the key stores read targets unconditionally: any valid [B][nkeys] array
    RoleArgs ar = role_for(L->fwd, xt, dyt, nullptr, dW, kWavesPerBlock, L->cap);
    ar.apply = apply;
    ar.lr = lr;
    const size_t lc = stream_lds_bytes(L->tr, p), lr_ = stream_lds_bytes(L->fwd, p);
    const size_t lds = lc > lr_ ? lc : lr_;
    const dim3 block(kLdsKeyWaves * kWave);
    // the column pass moves index + value in, value (or dW) out; the row pass index + value in, dW and value out
    const double bc = 10.0, br = apply ? 14.0 : 10.0;
    auto go = [&](auto kern) {
        int occ = 1;
        if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&occ, kern, (int)block.x, lds) != hipSuccess || occ < 1)
            occ = 1;
        int nwg = L->cus * (occ > 2 ? 2 : occ);
        nwg = (nwg + kXcd - 1) / kXcd * kXcd;
        int g0 = (int)(nwg * bc / (bc + br) + 0.5);
        if (g0 < 1) g0 = 1;
        if (g0 > nwg - 1) g0 = nwg - 1;
        hipLaunchKernelGGL(kern, dim3((unsigned)nwg), block, lds, s, ac, ar, g0, p.bp, B);
    };
    const bool i16 = L->tr.idx16 != nullptr && L->fwd.idx16 != nullptr;
    auto pick = [&](auto rmc, auto i16c, auto valc) {
        constexpr bool R = decltype(rmc)::value, I = decltype(i16c)::value, V = decltype(valc)::value;
        switch (p.btile) {
        case 1: go(stream_bwd_kernel<1, kStreamDepthFor<1>, R, I, V>); return true;
        case 2: go(stream_bwd_kernel<2, kStreamDepthFor<2>, R, I, V>); return true;
        case 4: go(stream_bwd_kernel<4, kStreamDepthFor<4>, R, I, V>); return true;
        default: return false;
        }
    };
    using T = std::true_type;
    using F = std::false_type;
    bool ok;
    if (apply) ok = rm ? (i16 ? pick(T{}, T{}, T{}) : pick(T{}, F{}, T{})) : (i16 ? pick(F{}, T{}, T{}) : pick(F{}, F{}, T{}));
    else ok = rm ? (i16 ? pick(T{}, T{}, F{}) : pick(T{}, F{}, F{})) : (i16 ? pick(F{}, T{}, F{}) : pick(F{}, F{}, F{}));
    if (!ok) return SNACK_ERR_INVALID_ARG;
    SNACK_HIP(hipGetLastError());
    return SNACK_OK;
}

// the split table of width index w of view v, valid: when it is stale, every
// stale table of the view is rebuilt in one pass over its index
snack_status ensure_split(const View& v, int w, hipStream_t s)
{
    if (v.split[w].S < 2 || v.split[w].valid) return SNACK_OK;
    TabSet ts;
    ts.inv_nidx = 1.0 / (double)v.nidx;
    for (int i = 0; i < kTileWidths; ++i) {
        const SplitTab& si = v.split[i];
        const bool build = si.S >= 2 && !si.valid;
        ts.S[i] = si.S;
        ts.tab[i] = build ? si.tab : nullptr;
    }
    hipLaunchKernelGGL(split_tables_kernel, dim3((unsigned)((v.nkeys + 3) / 4)), dim3(256), 0, s, v.ptr, v.idx,
                       v.nkeys, v.nidx, ts);
    SNACK_HIP(hipGetLastError());
    for (int i = 0; i < kTileWidths; ++i)
        if (ts.tab[i]) v.split[i].valid = true;
    return SNACK_OK;
}

inline int tile_index(int btile)
{
    return btile == 8 ? 0 : btile == 16 ? 1 : btile == 32 ? 2 : btile == 64 ? 3 : -1;
}

// slice-tiled kernels for batch tiles of 8 to 64 columns on long keys
// (use_tile: a single batch tile, for passes with dW; use_tile_spmm: passes
// without dW, which also take several 64-column tiles, one grid row each)
// key blocks per slice: about one workgroup per CU over all slices and batch
// tiles (each stages a whole slice, so with many tiles each workgroup takes
// more keys), at most 64 keys per wavefront
inline int tile_key_blocks(const snack_layer* L, const View& v, int S, int ntiles)
{
    const int64_t sweeps = (int64_t)S * ntiles;
    int kbn = (int)((L->cus + sweeps / 2) / sweeps);
    const int minkb = (v.nkeys + kTileWaves * 64 - 1) / (kTileWaves * 64);
    const int maxkb = (v.nkeys + kTileWaves - 1) / kTileWaves;
    if (kbn > maxkb) kbn = maxkb;
    if (kbn < minkb) kbn = minkb;
    return kbn < 1 ? 1 : kbn;
}

constexpr int64_t kTilePartMaxBytes = 256ll << 20;   // partial sums of all batch tiles at most
constexpr int64_t kTileMinEntries = 8192;            // entries per workgroup for several tiles
constexpr int64_t kTileMinKey64 = 32;                // average entries per key at the 64-column tile
inline bool use_tile_spmm(const snack_layer* L, const View& v, const BatchPlan& p)
{
    const int i = tile_index(p.btile);
    if (i < 0 || L->nnz <= 0 || v.split[i].S < 1) return false;
    // keys of 128 entries on average; at the 64-column tile also shorter ones (a
    // block's 16 entries carry 64 columns each, so short segments still pay)
    if (!use_keyed(v, L->nnz, p) && !(p.btile == 64 && v.nkeys > 0 && L->nnz / v.nkeys >= kTileMinKey64))
        return false;
    if (p.ntiles == 1) return true;
    // several tiles: every workgroup stages a slice once per tile, which pays only
    // when it has enough entries to walk
    const int S = v.split[i].S;
    return (int64_t)p.ntiles * S * v.nkeys * p.btile * 4 <= kTilePartMaxBytes &&
           L->nnz / ((int64_t)S * tile_key_blocks(L, v, S, p.ntiles)) >= kTileMinEntries;
}
inline bool use_tile(const snack_layer* L, const View& v, const BatchPlan& p)
{
    return p.ntiles == 1 && use_tile_spmm(L, v, p);
}

// dW in canonical order by its own pass over the row view (else permuted from
// the column pass's dW).  The two orders must agree bit for bit: up to batch
// tile 16 every kernel pair that can meet gives a lane the same columns and the
// same reduction; at 32 the tiled kernel interleaves a lane's columns and the
// key-major one does not, so both views must take the same family.
inline bool recompute_dw(const snack_layer* L, const BatchPlan& p)
{
    if (p.btile > kKeyedRecomputeMax || !use_keyed(L->fwd, L->nnz, p)) return false;
    return p.btile <= 16 || use_tile(L, L->tr, p) == use_tile(L, L->fwd, p);
}

// mse: the MSE gradient (and its feature-major copy) written by the slice
// reduction where there is one
template <bool DW, bool SPMM, bool VAL = false>
snack_status launch_tile(const BatchPlan& p, const snack_layer* L, const View& v, const float* G, const float* H,
                         float* out, float* dwo, int B, hipStream_t s, float* apply = nullptr, float lr = 0.0f,
                         MseFuse* mse = nullptr, float* part = nullptr)
{
    constexpr bool LV = SPMM || VAL;
    if (apply && !LV) return SNACK_ERR_INVALID_ARG;   // the step needs the values
    const SplitTab& st = v.split[tile_index(p.btile)];
    SNACK_CHECK(ensure_split(v, tile_index(p.btile), s));
    RoleArgs a = role_for(v, G, H, out, dwo, kWavesPerBlock, L->cap);
    a.apply = apply;
    a.lr = lr;
    TileArgs t;
    t.S = st.S;
    t.tab = st.S >= 2 ? st.tab : v.ptr;
    t.tstride = st.S >= 2 ? v.nkeys : 1;
    // over several batch tiles a dW pass writes one dW slab per tile (L->cap floats apart), to be
    // added up afterwards: no in-place step and no value-stepping row pass there
    if ((DW || VAL) && p.ntiles != 1 && (VAL || apply || !dwo)) return SNACK_ERR_INVALID_ARG;
    t.dwstride = p.ntiles != 1 ? L->cap : 0;
    // the slice partial sums: the layer's workspace unless the caller brings a buffer
    t.part = (st.S >= 2 && SPMM) ? (part ? part : ws_part(L, p)) : nullptr;
    t.pstride = (int64_t)t.S * v.nkeys * p.btile;
    const int kbn = tile_key_blocks(L, v, t.S, p.ntiles);
    t.KB = kbn;
    t.R = (v.nkeys + kbn - 1) / kbn;
    int64_t nwg = (int64_t)t.S * t.KB;
    nwg = (nwg + kXcd - 1) / kXcd * kXcd;
    const int32_t rows = (v.nidx + t.S - 1) / t.S + 1;   // the slice and a zero row
    const size_t lds = (size_t)rows * tile_row_floats(p.btile) * sizeof(float);
    const dim3 grid((unsigned)nwg, (unsigned)p.ntiles), block(kTileWaves * kWave);
    // group width x values per lane x entries per group: 2 x 4 x 2, 4 x 4 x 4,
    // 4 x 8 x 4, 16 x 4 x 8 (x 4 with dW: short slice segments waste less)
    constexpr int Dp = DW ? kTileDepthDw : kTileDepth;
    constexpr int U64 = DW ? 4 : 8;
    auto go = [&](auto kern) { hipLaunchKernelGGL(kern, grid, block, lds, s, a, t, p.bp, B); };
    switch (p.btile) {
    case 8: go(tile_kernel<2, 4, 2, Dp, DW, SPMM, LV>); break;
    case 16: go(tile_kernel<4, 4, 4, Dp, DW, SPMM, LV>); break;
    case 32: go(tile_kernel<4, 8, 4, Dp, DW, SPMM, LV>); break;
    case 64: go(tile_kernel<16, 4, U64, Dp, DW, SPMM, LV>); break;
    default: return SNACK_ERR_INVALID_ARG;
    }
    SNACK_HIP(hipGetLastError());
    if (t.part) {
        MseOut mo{nullptr, nullptr, nullptr, 0.0f};
        if (mse) {
            mo = MseOut{mse->T, mse->dY, mse->dYt, mse->scale};
            mse->done = true;
            mse->dyt_done = mse->dYt != nullptr;
        }
        auto rg = [&](int kpb) { return dim3((unsigned)((v.nkeys + kpb - 1) / kpb), (unsigned)p.ntiles); };
        switch (p.btile) {
        case 8:
            hipLaunchKernelGGL((split_reduce_kernel<8>), rg(kSplitReduceKeys<8>), dim3(256), 0, s, t.part, t.S, v.nkeys,
                               B, out, mo);
            break;
        case 16:
            hipLaunchKernelGGL((split_reduce_kernel<16>), rg(kSplitReduceKeys<16>), dim3(256), 0, s, t.part, t.S,
                               v.nkeys, B, out, mo);
            break;
        case 32:
            hipLaunchKernelGGL((split_reduce_kernel<32>), rg(kSplitReduceKeys<32>), dim3(256), 0, s, t.part, t.S,
                               v.nkeys, B, out, mo);
            break;
        default:
            hipLaunchKernelGGL((split_reduce_kernel<64>), rg(kSplitReduceKeys<64>), dim3(256), 0, s, t.part, t.S,
                               v.nkeys, B, out, mo);
            break;
        }
        SNACK_HIP(hipGetLastError());
    }
    return SNACK_OK;
}

// The backward's two slice-tiled passes at one batch tile in one launch (see
// tile_bwd_kernel), then the column pass's slice reduction into dX.  The
// column pass steps vals_t and writes no dW; the row pass writes the canonical
// dW and steps vals.
snack_status launch_tile_bwd2(const BatchPlan& p, const snack_layer* L, const float* dyt, const float* xt, float* dX,
                              float* dW, float lr, int B, hipStream_t s)
{
    if (p.ntiles != 1) return SNACK_ERR_INVALID_ARG;
    const int w = tile_index(p.btile);
    SNACK_CHECK(ensure_split(L->tr, w, s));
    SNACK_CHECK(ensure_split(L->fwd, w, s));
    auto setup = [&](const View& v, const float* G, const float* H, float* out, float* dwo, float* apply, bool spmm,
                     RoleArgs& a, TileArgs& t, int64_t& nwg, size_t& lds) {
        const SplitTab& st = v.split[w];
        a = role_for(v, G, H, out, dwo, kWavesPerBlock, L->cap);
        a.apply = apply;
        a.lr = lr;
        t.S = st.S;
        t.tab = st.S >= 2 ? st.tab : v.ptr;
        t.tstride = st.S >= 2 ? v.nkeys : 1;
        t.dwstride = 0;
        t.part = (st.S >= 2 && spmm) ? ws_part(L, p) : nullptr;
        t.pstride = (int64_t)t.S * v.nkeys * p.btile;
        t.KB = tile_key_blocks(L, v, t.S, p.ntiles);
        t.R = (v.nkeys + t.KB - 1) / t.KB;
        nwg = (int64_t)t.S * t.KB;
        nwg = (nwg + kXcd - 1) / kXcd * kXcd;
        const int32_t rows = (v.nidx + t.S - 1) / t.S + 1;   // the slice and a zero row
        lds = (size_t)rows * tile_row_floats(p.btile) * sizeof(float);
    };
    RoleArgs ac, ar;
    TileArgs tc, tr;
    int64_t nc, nr;
    size_t lc, lr_;
    setup(L->tr, dyt, xt, dX, nullptr, L->vals_t, true, ac, tc, nc, lc);
    setup(L->fwd, xt, dyt, nullptr, dW, L->vals, false, ar, tr, nr, lr_);
    const size_t lds = lc > lr_ ? lc : lr_;
    const dim3 grid((unsigned)(nc + nr), 1), block(kTileWaves * kWave);
    constexpr int Dp = kTileDepthDw;
    auto go = [&](auto kern) { hipLaunchKernelGGL(kern, grid, block, lds, s, ac, tc, ar, tr, (int)nc, p.bp, B); };
    switch (p.btile) {
    case 8: go(tile_bwd_kernel<2, 4, 2, Dp>); break;
    case 16: go(tile_bwd_kernel<4, 4, 4, Dp>); break;
    case 32: go(tile_bwd_kernel<4, 8, 4, Dp>); break;
    case 64: go(tile_bwd_kernel<16, 4, 4, Dp>); break;
    default: return SNACK_ERR_INVALID_ARG;
    }
    SNACK_HIP(hipGetLastError());
    if (tc.part) {
        const MseOut mo{nullptr, nullptr, nullptr, 0.0f};
        const View& v = L->tr;
        auto rg = [&](int kpb) { return dim3((unsigned)((v.nkeys + kpb - 1) / kpb), 1u); };
        switch (p.btile) {
        case 8:
            hipLaunchKernelGGL((split_reduce_kernel<8>), rg(kSplitReduceKeys<8>), dim3(256), 0, s, tc.part, tc.S,
                               v.nkeys, B, dX, mo);
            break;
        case 16:
            hipLaunchKernelGGL((split_reduce_kernel<16>), rg(kSplitReduceKeys<16>), dim3(256), 0, s, tc.part, tc.S,
                               v.nkeys, B, dX, mo);
            break;
        case 32:
            hipLaunchKernelGGL((split_reduce_kernel<32>), rg(kSplitReduceKeys<32>), dim3(256), 0, s, tc.part, tc.S,
                               v.nkeys, B, dX, mo);
            break;
        default:
            hipLaunchKernelGGL((split_reduce_kernel<64>), rg(kSplitReduceKeys<64>), dim3(256), 0, s, tc.part, tc.S,
                               v.nkeys, B, dX, mo);
            break;
        }
        SNACK_HIP(hipGetLastError());
    }
    return SNACK_OK;
}

}  // namespace

int tile_splits(const snack_layer* L, const View& v, int btile)
{
    if (L->lds_bytes <= kTileStaticLds || v.nidx <= 0 || v.nkeys <= 0) return 0;
    const int64_t rows = (int64_t)(L->lds_bytes - kTileStaticLds) / ((int64_t)tile_row_floats(btile) * 4);
    if (rows < 1) return 0;
    const int64_t S = (v.nidx + rows - 1) / rows;
    return S <= kMaxSplits ? (int)S : 0;
}

snack_status alloc_split_tables(snack_layer* L)
{
    View* views[2] = {&L->fwd, &L->tr};
    for (View* v : views) {
        for (int i = 0; i < kTileWidths; ++i) {
            SplitTab& st = v->split[i];
            st.S = tile_splits(L, *v, 8 << i);
            st.tab = nullptr;
            st.valid = false;
            if (st.S >= 2) {
                void* q = nullptr;
                SNACK_CHECK(layer_alloc(L, &q, (size_t)(st.S + 1) * v->nkeys * sizeof(int32_t)));
                st.tab = (int32_t*)q;
            }
        }
    }
    return SNACK_OK;
}

size_t forward_part_bytes(const snack_layer* L, const BatchPlan& p)
{
    if (!use_tile_spmm(L, L->fwd, p)) return 0;
    const SplitTab& st = L->fwd.split[tile_index(p.btile)];
    if (st.S < 2) return 0;
    const size_t b = (size_t)p.ntiles * st.S * L->fwd.nkeys * p.btile * sizeof(float);
    return (b + 255) & ~(size_t)255;
}

size_t tile_part_bytes(const snack_layer* L, const BatchPlan& p)
{
    size_t need = 0;
    const View* views[2] = {&L->fwd, &L->tr};
    for (const View* v : views) {
        if (!use_tile_spmm(L, *v, p)) continue;
        const SplitTab& st = v->split[tile_index(p.btile)];
        if (st.S < 2) continue;
        const size_t b = (size_t)p.ntiles * st.S * v->nkeys * p.btile * sizeof(float);
        if (b > need) need = b;
    }
    return (need + 255) & ~(size_t)255;
}

BatchPlan plan_batch(int B)
{
    BatchPlan p;
    if (B <= 1) { p.bt = 1; p.nb = 1; }
    else if (B == 2) { p.bt = 1; p.nb = 2; }
    else if (B <= 4) { p.bt = 1; p.nb = 4; }
    else if (B <= 8) { p.bt = 1; p.nb = 8; }
    else if (B <= 16) { p.bt = 2; p.nb = 8; }
    else if (B <= 32) { p.bt = 4; p.nb = 8; }
    else { p.bt = 8; p.nb = 8; }
    p.u = 4;
    p.btile = p.bt * p.nb;
    p.ntiles = (B + p.btile - 1) / p.btile;
    p.bp = p.ntiles * p.btile;
    return p;
}

// The tiled permutation for width index w: the tiles of the width-w split
// tables of both views, when there are enough of them and an average tile's
// entries (with a margin) fit in LDS; false when it does not apply.
static bool perm_tiles_plan(const snack_layer* L, int w, PermArgs* P, size_t* lds)
{
    if (L->nnz <= 0 || w < 0 || L->tr.split[w].S < 2 || L->fwd.split[w].S < 2) return false;
    P->SA = L->tr.split[w].S;
    P->SB = L->fwd.split[w].S;
    P->M = L->M;
    P->K = L->K;
    P->nrmax = (L->M + P->SA - 1) / P->SA + 1;
    P->ncmax = (L->K + P->SB - 1) / P->SB + 1;
    const int64_t tiles = (int64_t)P->SA * P->SB;
    const int64_t tables = (int64_t)(2 * P->nrmax + 2 * P->ncmax + 1) * 4;
    const int64_t budget = (int64_t)L->lds_bytes - 1024 - tables;
    const double avg = (double)L->nnz / (double)tiles;
    const int64_t want = (int64_t)(avg * 1.25) + 1024;
    if (tiles < 64 || budget / 4 < want) return false;
    P->cap = (int32_t)want;
    *lds = (size_t)want * 4 + (size_t)tables;
    return true;
}

// dW[k] = dW_t[iperm[k]], by tiles where perm_tiles_plan allows
static snack_status permute_dw(const snack_layer* L, int w, const float* dW_t, float* dW, hipStream_t s)
{
    {
        PermArgs P;
        size_t lds = 0;
        if (perm_tiles_plan(L, w, &P, &lds)) {
            const int64_t tiles = (int64_t)P.SA * P.SB;
            SNACK_CHECK(ensure_split(L->tr, w, s));
            SNACK_CHECK(ensure_split(L->fwd, w, s));
            P.ttab = L->tr.split[w].tab;
            P.ts = L->tr.nkeys;
            P.ftab = L->fwd.split[w].tab;
            P.fs = L->fwd.nkeys;
            P.iperm = L->iperm;
            P.cols = L->cols;
            P.dwt = dW_t;
            P.dw = dW;
            hipLaunchKernelGGL(permute_tiles_kernel, dim3((unsigned)tiles), dim3(kPermThreads), lds, s, P);
            SNACK_HIP(hipGetLastError());
            return SNACK_OK;
        }
    }
    if (L->nnz > 0) {
        const int64_t per_xcd = (L->nnz + kXcd - 1) / kXcd;
        int64_t nw = (per_xcd + kBlock - 1) / kBlock;
        if (nw > 256) nw = 256;   // about eight resident workgroups per CU
        hipLaunchKernelGGL(permute_dw_kernel, dim3((unsigned)(nw * kXcd)), dim3(kBlock), 0, s, L->iperm, dW_t, L->nnz,
                           per_xcd, dW);
        SNACK_HIP(hipGetLastError());
    }
    return SNACK_OK;
}

bool spmm_batch_major(const snack_layer* L, const BatchPlan& p, bool fwd, bool dx, bool dw)
{
    if (p.bp <= 1) return false;   // one column: both layouts coincide
    if (fwd) return keyed_lds(L, L->fwd, p);
    if (dw && !dx) return keyed_lds(L, L->fwd, p);
    if (dx && !dw) return keyed_lds(L, L->tr, p);
    // dX and dW: the column pass, then dW recomputed over the row view
    return dx && dw && p.btile <= kKeyedRecomputeMax && keyed_lds(L, L->tr, p) && keyed_lds(L, L->fwd, p);
}

snack_status spmm_forward(const snack_layer* L, const float* feat_t, const BatchPlan& p, int B, float* out,
                          hipStream_t s, bool rm, MseFuse* mse, float* part)
{
    ProfScope prof(KC_SPMM_FWD, s);
    if (rm) return launch_keyed<false>(p, L, L->fwd, feat_t, nullptr, out, nullptr, B, s, true, nullptr, 0.0f, mse);
    if (wide_short(L, L->fwd, p)) return wide_spmm(L, L->fwd, feat_t, p, B, out, s);
    if (use_tile_spmm(L, L->fwd, p))
        return launch_tile<false, true>(p, L, L->fwd, feat_t, nullptr, out, nullptr, B, s, nullptr, 0.0f, mse, part);
    if (use_keyed(L->fwd, L->nnz, p) || keyed_lds(L, L->fwd, p))
        return launch_keyed<false>(p, L, L->fwd, feat_t, nullptr, out, nullptr, B, s, false, nullptr, 0.0f, mse);
    return dispatch_seg<false>(p, L->cap, L->fwd, feat_t, nullptr, out, nullptr, nullptr, nullptr, nullptr, nullptr,
                               B, s);
}

bool infer_supported(const snack_layer* L, int B, bool b16)
{
    const BatchPlan p = plan_batch(B);
    return p.ntiles == 1 && p.btile <= 4 && keyed_lds(L, L->fwd, p) && (!b16 || (L->fwd.idx16 && L->vals16));
}

snack_status spmm_forward_infer(const snack_layer* L, const float* X, float* Y, int B, int act, bool b16,
                                hipStream_t s)
{
    if (!infer_supported(L, B, b16)) return SNACK_ERR_UNSUPPORTED;
    ProfScope prof(KC_SPMM_FWD, s);
    const BatchPlan p = plan_batch(B);
    const bool rm = p.bp > 1;   // one column: both layouts coincide
    RoleArgs a = role_for(L->fwd, X, nullptr, Y, nullptr, kWavesPerBlock, L->cap);
    a.tgt = Y;
    a.act = act;
    a.vals16 = b16 ? L->vals16 : nullptr;
    const size_t lds = stream_lds_bytes(L->fwd, p);
    const dim3 block(kLdsKeyWaves * kWave);
    auto go = [&](auto kern) {
        int occ = 1;
        if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&occ, kern, (int)block.x, lds) != hipSuccess || occ < 1)
            occ = 1;
        int nwg = L->cus * (occ > 2 ? 2 : occ);
        const int want = (L->fwd.nkeys + kLdsKeyWaves - 1) / kLdsKeyWaves;
        if (nwg > want) nwg = want;
        nwg = (nwg + kXcd - 1) / kXcd * kXcd;
        hipLaunchKernelGGL(kern, dim3((unsigned)nwg), block, lds, s, a, p.bp, B);
    };
    const bool i16 = L->fwd.idx16 != nullptr;
    auto pick = [&](auto rmc, auto i16c, auto v16c) {
        constexpr bool R = decltype(rmc)::value, I = decltype(i16c)::value, V = decltype(v16c)::value;
        switch (p.btile) {
        case 1: go(stream_lds_kernel<1, kStreamDepthFor<1>, false, true, R, true, I, V>); return true;
        case 2: go(stream_lds_kernel<2, kStreamDepthFor<2>, false, true, R, true, I, V>); return true;
        case 4: go(stream_lds_kernel<4, kStreamDepthFor<4>, false, true, R, true, I, V>); return true;
        default: return false;
        }
    };
    using T = std::true_type;
    using F = std::false_type;
    bool ok;
    if (b16) ok = rm ? pick(T{}, T{}, T{}) : pick(F{}, T{}, T{});
    else ok = rm ? (i16 ? pick(T{}, T{}, F{}) : pick(T{}, F{}, F{})) : (i16 ? pick(F{}, T{}, F{}) : pick(F{}, F{}, F{}));
    if (!ok) return SNACK_ERR_INVALID_ARG;
    SNACK_HIP(hipGetLastError());
    return SNACK_OK;
}

snack_status spmm_backward_fused(const snack_layer* L, const float* xt, const float* dyt, const BatchPlan& p, int B,
                                 float* dX, float* dW, float* dW_t, hipStream_t s, bool rm, SgdStep* step)
{
    // the in-place step of vals_t by the column pass that also yields dW (single batch tile), for the
    // batch-major passes (the slice-tiled and key-major passes decide below)
    float* apply = (step && dX && dW && p.ntiles == 1 && p.btile <= 32) ? L->vals_t : nullptr;
    const float lr = step ? step->lr : 0.0f;
    if (dX && dW && p.ntiles == 1 && p.btile <= 4 && keyed_lds(L, L->tr, p) && keyed_lds(L, L->fwd, p)) {
        // both passes in one launch of the two-role streamed kernel (counted as the column pass); with
        // the step both value copies are stepped in place and no column-order dW is written
        ProfScope prof(KC_SPMM_DX, s);
        SNACK_CHECK(launch_stream_bwd(p, L, dyt, xt, dX, step ? nullptr : dW_t, step ? L->vals_t : nullptr, dW,
                                      step ? L->vals : nullptr, lr, B, s, rm));
        if (step) {
            step->done = true;
            step->canon_done = true;
        }
        return SNACK_OK;
    }
    if (rm) {
        // batch-major operands: every pass is the LDS key-major kernel
        if (dW && !dX) {
            ProfScope prof(KC_SDDMM_DW, s);
            return launch_keyed<true, false>(p, L, L->fwd, xt, dyt, nullptr, dW, B, s, true);
        }
        if (dX && !dW) {
            ProfScope prof(KC_SPMM_DX, s);
            return launch_keyed<false>(p, L, L->tr, dyt, xt, dX, nullptr, B, s, true);
        }
        if (!dW_t && !apply) return SNACK_ERR_INVALID_ARG;
        {
            // the canonical dW is recomputed below, so with the step the column order needs no dW of its own
            ProfScope prof(KC_SPMM_DX, s);
            SNACK_CHECK(launch_keyed<true>(p, L, L->tr, dyt, xt, dX, apply ? nullptr : dW_t, B, s, true, apply, lr));
        }
        ProfScope prof(KC_SDDMM_DW, s);
        if (!apply) return launch_keyed<true, false>(p, L, L->fwd, xt, dyt, nullptr, dW, B, s, true);
        // the row pass steps the canonical values in place from the dW it computes
        SNACK_CHECK((launch_keyed<true, false, true>(p, L, L->fwd, xt, dyt, nullptr, dW, B, s, true, L->vals, lr)));
        step->done = true;
        step->canon_done = true;
        return SNACK_OK;
    }
    // role A: dX (and dW in column order) over the transposed view; role B: dW over the canonical view.
    // Event classes: the column pass counts as dX, a separate canonical-order dW step as dW.
    if (dW && !dX) {
        ProfScope prof(KC_SDDMM_DW, s);
        if (p.ntiles == 1 && (use_keyed(L->fwd, L->nnz, p) || keyed_lds(L, L->fwd, p)))
            return launch_keyed<true, false>(p, L, L->fwd, xt, dyt, nullptr, dW, B, s);
        return dispatch_seg<true>(p, L->cap, L->fwd, xt, dyt, nullptr, dW, nullptr, nullptr, nullptr, nullptr, B, s);
    }
    if (dW && dW_t && p.ntiles == 1 && use_keyed(L->tr, L->nnz, p)) {
        const bool recompute = recompute_dw(L, p);
        if (step && recompute && use_tile(L, L->tr, p) && use_tile(L, L->fwd, p)) {
            // both slice-tiled passes in one launch (counted as the column pass), each stepping its values
            ProfScope prof(KC_SPMM_DX, s);
            SNACK_CHECK(launch_tile_bwd2(p, L, dyt, xt, dX, dW, step->lr, B, s));
            step->done = true;
            step->canon_done = true;
            return SNACK_OK;
        }
        // with the step the column pass steps vals_t in place; where the canonical dW is permuted from the
        // column order, the canonical values then take their step in a separate pass (cheaper than in the
        // permutation, which waits on memory)
        float* ap = step ? L->vals_t : nullptr;
        {
            // with the step, dW in column order is still needed where the canonical dW is permuted from it
            float* dwo = (ap && recompute) ? nullptr : dW_t;
            ProfScope prof(KC_SPMM_DX, s);
            if (use_tile(L, L->tr, p))
                SNACK_CHECK((launch_tile<true, true>(p, L, L->tr, dyt, xt, dX, dwo, B, s, ap, lr)));
            else SNACK_CHECK(launch_keyed<true>(p, L, L->tr, dyt, xt, dX, dwo, B, s, false, ap, lr));
            if (ap) step->done = true;
        }
        ProfScope prof(KC_SDDMM_DW, s);
        if (recompute) {
            // narrow batches: dW in canonical order by a second (cheap) pass over the row view, which
            // with the step also steps the canonical values in place
            if (!ap) {
                if (use_tile(L, L->fwd, p)) return launch_tile<true, false>(p, L, L->fwd, xt, dyt, nullptr, dW, B, s);
                return launch_keyed<true, false>(p, L, L->fwd, xt, dyt, nullptr, dW, B, s);
            }
            if (use_tile(L, L->fwd, p))
                SNACK_CHECK((launch_tile<true, false, true>(p, L, L->fwd, xt, dyt, nullptr, dW, B, s, L->vals, lr)));
            else SNACK_CHECK((launch_keyed<true, false, true>(p, L, L->fwd, xt, dyt, nullptr, dW, B, s, false, L->vals,
                                                               lr)));
            step->canon_done = true;
            return SNACK_OK;
        }
        // wide batches: dW once, in column order, then permuted into canonical order
        return permute_dw(L, tile_index(p.btile), dW_t, dW, s);
    }
    ProfScope prof(KC_SPMM_DX, s);
    if (dW)
        return dispatch_seg<true>(p, L->cap, L->tr, dyt, xt, dX, dW_t, &L->fwd, xt, dyt, dW, B, s);
    if (use_tile_spmm(L, L->tr, p)) return launch_tile<false, true>(p, L, L->tr, dyt, xt, dX, nullptr, B, s);
    if (use_keyed(L->tr, L->nnz, p) || keyed_lds(L, L->tr, p))
        return launch_keyed<false>(p, L, L->tr, dyt, xt, dX, nullptr, B, s);
    return dispatch_seg<true>(p, L->cap, L->tr, dyt, xt, dX, dW_t, nullptr, nullptr, nullptr, nullptr, B, s);
}

namespace {

// dW in column order from the per-tile slabs: dwt[e] = sum over tiles, in tile order
__global__ void dw_slab_sum_kernel(const float* __restrict__ slabs, int64_t stride, int ntiles, int64_t nnz,
                                   float* __restrict__ dwt)
{
    const int64_t n4 = nnz >> 2;
    const int64_t step = (int64_t)gridDim.x * blockDim.x;
    for (int64_t q = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; q < n4; q += step) {
        float4 a = *reinterpret_cast<const float4*>(slabs + 4 * q);
        for (int t = 1; t < ntiles; ++t) {
            const float4 b = *reinterpret_cast<const float4*>(slabs + (int64_t)t * stride + 4 * q);
            a.x += b.x;
            a.y += b.y;
            a.z += b.z;
            a.w += b.w;
        }
        *reinterpret_cast<float4*>(dwt + 4 * q) = a;
    }
    for (int64_t e = 4 * n4 + (int64_t)blockIdx.x * blockDim.x + threadIdx.x; e < nnz; e += step) {
        float a = slabs[e];
        for (int t = 1; t < ntiles; ++t) a += slabs[(int64_t)t * stride + e];
        dwt[e] = a;
    }
}

}  // namespace

bool wide_dw_fused(const snack_layer* L, const BatchPlan& p)
{
    return p.ntiles > 1 && p.btile == 64 && L->nnz > 0 && L->cap % 4 == 0 &&
           (int64_t)p.ntiles * L->cap * 4 <= kTilePartMaxBytes && use_tile_spmm(L, L->tr, p);
}

size_t wide_dw_bytes(const snack_layer* L, const BatchPlan& p)
{
    return wide_dw_fused(L, p) ? (((size_t)p.ntiles * L->cap * 4) + 255) & ~(size_t)255 : 0;
}

snack_status spmm_backward_wide(const snack_layer* L, const float* xt, const float* dyt, const BatchPlan& p, int B,
                                float* dX, float* dW, float* dW_t, float* slabs, hipStream_t s)
{
    if (!wide_dw_fused(L, p) || !dX || !dW || !dW_t || !slabs) return SNACK_ERR_INVALID_ARG;
    {
        ProfScope prof(KC_SPMM_DX, s);
        SNACK_CHECK((launch_tile<true, true>(p, L, L->tr, dyt, xt, dX, slabs, B, s)));
    }
    ProfScope prof(KC_SDDMM_DW, s);
    const int64_t n4 = (L->nnz + 3) / 4;
    const unsigned grid = (unsigned)std::min<int64_t>((n4 + 255) / 256, 4096);
    hipLaunchKernelGGL(dw_slab_sum_kernel, dim3(grid), dim3(256), 0, s, slabs, L->cap, p.ntiles, L->nnz, dW_t);
    SNACK_HIP(hipGetLastError());
    return permute_dw(L, tile_index(p.btile), dW_t, dW, s);
}

snack_status sddmm_dw_tiles(const snack_layer* L, const float* xt, const float* dyt, const BatchPlan& p, float* dW,
                            hipStream_t s)
{
    if (L->nnz == 0) return SNACK_OK;
    ProfScope prof(KC_SDDMM_DW, s);
    constexpr int BT = 8, NB = 8, U = 4;
    if (p.bt != BT || p.nb != NB) return SNACK_ERR_INVALID_ARG;
    constexpr int STEP = (kWave / BT) * U;
    const int64_t nsteps = (L->nnz + STEP - 1) / STEP;
    int64_t nb = (nsteps + kWavesPerBlock - 1) / kWavesPerBlock;
    if (nb > 256 * 16) nb = 256 * 16;
    hipLaunchKernelGGL((sddmm_tiles_kernel<BT, NB, U>), dim3((unsigned)nb), dim3(kBlock), 0, s, L->rows, L->cols,
                       L->nnz, xt, dyt, p.bp, p.ntiles, dW, nsteps);
    SNACK_HIP(hipGetLastError());
    return SNACK_OK;
}

}  // namespace snack
