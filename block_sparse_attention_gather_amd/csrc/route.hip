// Sparse-routing frontend (FVAttn page, abstract: Top-p routing with a Top-k safety floor over
// video-aware blocks, producing a materialized block mask).
//
//   pool   : qbar_j, kbar_j = mean of the tiled Q / K rows of block j over its real tokens,
//            fp64 (sums of bf16 values are exact in fp64 for the value ranges involved).
//   route  : s_ij = scale * <qbar_i, kbar_j> in fp64 for R query blocks of one head per
//            workgroup (k-bar rows read once per R rows), then per row: bitonic sort of
//            (s desc, j asc) in LDS, block softmax mass in sorted order, prefix sum, Top-p cut,
//            Top-k floor, and a kept-block bitmap + count written to the workspace.
//   scan   : exclusive scan of the per-row counts -> CSR row_ptr and nnz.
//   fill   : bitmap -> ascending column list at col_idx[row_ptr[r]...] (one wavefront a row).
//
// Bounds: memory-bound (pool reads Q and K once); the fp64 scoring is ~2*n_blk^2*D flop per
// head, small next to the attention.
#include "bsa_internal.h"

namespace bsa {
namespace {

constexpr int kThreads = 256;

__device__ __forceinline__ double bf16_lo(uint32_t w) { return (double)__uint_as_float(w << 16); }
__device__ __forceinline__ double bf16_hi(uint32_t w) {
    return (double)__uint_as_float(w & 0xffff0000u);
}

// ---------------------------------------------------------------------------------------
// pool: grid (n_blk, batch*heads, 2)
// ---------------------------------------------------------------------------------------
template <int D>
__global__ __launch_bounds__(kThreads) void pool_kernel(const uint4* __restrict__ q,
                                                        const uint4* __restrict__ k,
                                                        double* __restrict__ qbar,
                                                        double* __restrict__ kbar, int64_t N,
                                                        int64_t Npad, int32_t B,
                                                        int32_t n_blk) {
    constexpr int DCH = D / 8;              // 16-byte chunks per row
    constexpr int RPP = kThreads / DCH;     // rows per pass
    __shared__ double red[RPP][D + 1];
    const int t = threadIdx.x;
    const int dc = t % DCH, rp = t / DCH;
    const int32_t j = blockIdx.x;
    const int64_t bh = blockIdx.y;
    const uint4* src = (blockIdx.z == 0 ? q : k) + bh * Npad * DCH;
    double* out = (blockIdx.z == 0 ? qbar : kbar) + (bh * n_blk + j) * D;
    const int64_t lo = (int64_t)j * B;
    const int64_t hi = min(lo + B, N);
    double acc[8];
#pragma unroll
    for (int e = 0; e < 8; ++e) acc[e] = 0.0;
    for (int64_t p = lo + rp; p < hi; p += RPP) {
        const uint4 v = src[p * DCH + dc];
        acc[0] += bf16_lo(v.x); acc[1] += bf16_hi(v.x);
        acc[2] += bf16_lo(v.y); acc[3] += bf16_hi(v.y);
        acc[4] += bf16_lo(v.z); acc[5] += bf16_hi(v.z);
        acc[6] += bf16_lo(v.w); acc[7] += bf16_hi(v.w);
    }
#pragma unroll
    for (int e = 0; e < 8; ++e) red[rp][dc * 8 + e] = acc[e];
    __syncthreads();
    for (int d = t; d < D; d += kThreads) {
        double s = 0.0;
        for (int r = 0; r < RPP; ++r) s += red[r][d];
        out[d] = s / (double)(hi - lo);
    }
}

// ---------------------------------------------------------------------------------------
// route: grid (ceil(n_blk / R), batch*heads); dynamic LDS (see route_lds_bytes)
// ---------------------------------------------------------------------------------------
__device__ __forceinline__ uint64_t desc_key(double s) {
    // ascending key order == descending score order; -0.0 and +0.0 map to one key
    const double ns = -s + 0.0;
    const uint64_t b = (uint64_t)__double_as_longlong(ns);
    return (b >> 63) ? ~b : (b | 0x8000000000000000ull);
}

struct RouteArgs {
    const double* qbar;
    const double* kbar;
    uint32_t* bitmap;       // [rows][nwords]
    int32_t* counts;        // [rows]
    double* scores_out;     // optional [rows][n_blk]
    double scale;
    double top_p;
    int32_t k_floor;
    int32_t n_blk;
    int32_t P2;             // power of two >= n_blk
    int32_t R;              // query blocks per workgroup (<= 8)
    int32_t nwords;         // ceil(n_blk / 32)
};

static size_t route_lds_bytes(int D, int P2, int R) {
    return (size_t)R * P2 * 8       // scores
           + (size_t)P2 * 8          // sort keys
           + (size_t)P2 * 4          // sort indices
           + (size_t)kThreads * 8    // scan / reduction scratch
           + (size_t)(P2 / 32 + 1) * 4  // bitmap
           + (size_t)R * D * 8;      // pooled queries
}

__device__ double block_sum(double v, double* scratch) {
    const int t = threadIdx.x;
    scratch[t] = v;
    __syncthreads();
    for (int off = kThreads / 2; off > 0; off >>= 1) {
        if (t < off) scratch[t] += scratch[t + off];
        __syncthreads();
    }
    const double r = scratch[0];
    __syncthreads();
    return r;
}

template <int D>
__global__ __launch_bounds__(kThreads) void route_kernel(RouteArgs a) {
    extern __shared__ __align__(16) unsigned char smem[];
    const int t = threadIdx.x;
    const int P2 = a.P2, R = a.R, n = a.n_blk;
    double* sc = (double*)smem;                               // [R][P2]
    uint64_t* key = (uint64_t*)(sc + (size_t)R * P2);          // [P2]
    uint32_t* idx = (uint32_t*)(key + P2);                     // [P2]
    double* scratch = (double*)(idx + P2);                     // [kThreads]
    uint32_t* bits = (uint32_t*)(scratch + kThreads);          // [P2/32 + 1]
    double* qb = (double*)(bits + (P2 / 32 + 1) + ((P2 / 32 + 1) & 1));  // [R][D], 8B aligned

    const int64_t bh = blockIdx.y;
    const int32_t i0 = blockIdx.x * R;
    const int32_t nr = min(R, n - i0);
    const double* qbar = a.qbar + (bh * n + i0) * D;
    const double* kbar = a.kbar + bh * n * D;

    for (int e = t; e < nr * D; e += kThreads) qb[e] = qbar[e];
    __syncthreads();

    // scores for the nr rows of this workgroup
    for (int j = t; j < n; j += kThreads) {
        double acc[8];
#pragma unroll
        for (int r = 0; r < 8; ++r) acc[r] = 0.0;
        const double2* kr = (const double2*)(kbar + (int64_t)j * D);
        for (int d2 = 0; d2 < D / 2; ++d2) {
            const double2 kv = kr[d2];
#pragma unroll
            for (int r = 0; r < 8; ++r) {
                if (r < nr) {
                    acc[r] = fma(qb[r * D + 2 * d2], kv.x, acc[r]);
                    acc[r] = fma(qb[r * D + 2 * d2 + 1], kv.y, acc[r]);
                }
            }
        }
#pragma unroll
        for (int r = 0; r < 8; ++r) {
            if (r < nr) {
                const double s = a.scale * acc[r];
                sc[r * P2 + j] = s;
                if (a.scores_out) a.scores_out[(bh * n + i0 + r) * (int64_t)n + j] = s;
            }
        }
    }
    __syncthreads();

    const int seg = (P2 + kThreads - 1) / kThreads;   // positions per thread in the scan
    for (int r = 0; r < nr; ++r) {
        const double* s = sc + r * P2;
        for (int e = t; e < P2; e += kThreads) {
            key[e] = e < n ? desc_key(s[e]) : ~0ull;
            idx[e] = e < n ? (uint32_t)e : 0xffffffffu;
        }
        for (int e = t; e < P2 / 32 + 1; e += kThreads) bits[e] = 0u;
        __syncthreads();
        // bitonic sort, ascending on (key, idx)
        for (int kk = 2; kk <= P2; kk <<= 1) {
            for (int jj = kk >> 1; jj > 0; jj >>= 1) {
                for (int e = t; e < P2 / 2; e += kThreads) {
                    const int lo = ((e & ~(jj - 1)) << 1) | (e & (jj - 1));
                    const int hi = lo + jj;
                    const uint64_t ka = key[lo], kb = key[hi];
                    const uint32_t ia = idx[lo], ib = idx[hi];
                    const bool a_gt_b = (ka > kb) || (ka == kb && ia > ib);
                    const bool up = (lo & kk) == 0;
                    if (a_gt_b == up) {
                        key[lo] = kb; key[hi] = ka;
                        idx[lo] = ib; idx[hi] = ia;
                    }
                }
                __syncthreads();
            }
        }
        // block mass along the sorted order; the first sorted entry holds the row maximum
        const double smax = s[idx[0]];
        const int p0 = t * seg;
        double local = 0.0;
        for (int u = 0; u < seg; ++u) {
            const int pos = p0 + u;
            if (pos < n) local += exp(s[idx[pos]] - smax);
        }
        const double Z = block_sum(local, scratch);
        // inclusive scan of the normalized mass: thread-segment totals, then a block scan
        double segsum = 0.0;
        for (int u = 0; u < seg; ++u) {
            const int pos = p0 + u;
            if (pos < n) segsum += exp(s[idx[pos]] - smax) / Z;
        }
        scratch[t] = segsum;
        __syncthreads();
        for (int off = 1; off < kThreads; off <<= 1) {
            const double add = t >= off ? scratch[t - off] : 0.0;
            __syncthreads();
            scratch[t] += add;
            __syncthreads();
        }
        double cum = scratch[t] - segsum;      // exclusive prefix of this segment
        __syncthreads();
        int first = n;                          // first sorted position with cum >= top_p
        for (int u = 0; u < seg; ++u) {
            const int pos = p0 + u;
            if (pos < n) {
                cum += exp(s[idx[pos]] - smax) / Z;
                if (first == n && cum >= a.top_p) first = pos;
            }
        }
        // block min of `first`
        scratch[t] = (double)first;
        __syncthreads();
        for (int off = kThreads / 2; off > 0; off >>= 1) {
            if (t < off) scratch[t] = fmin(scratch[t], scratch[t + off]);
            __syncthreads();
        }
        int kp;
        if (a.top_p >= 1.0) kp = n;
        else if (a.top_p <= 0.0) kp = 0;
        else kp = scratch[0] < (double)n ? (int)scratch[0] + 1 : n;
        __syncthreads();
        const int c = min(n, max(kp, a.k_floor));
        for (int pos = t; pos < c; pos += kThreads) {
            const uint32_t j = idx[pos];
            atomicOr(&bits[j >> 5], 1u << (j & 31));
        }
        __syncthreads();
        const int64_t row = bh * n + i0 + r;
        for (int w = t; w < a.nwords; w += kThreads) a.bitmap[row * a.nwords + w] = bits[w];
        if (t == 0) a.counts[row] = c;
        __syncthreads();
    }
}


// ---------------------------------------------------------------------------------------
// score: S[bh][i][j] = scale * <qbar_i, kbar_j>, fp64 MFMA 16x16x4 (rows of up to 2048 blocks).
// 1-D grid of 8 * T * ceil(bh / 8) workgroups, T = ceil(n/64)^2 tiles of 64 x 64 per head:
// workgroup L runs on XCD L % 8 and takes tile (L / 8) % T of head L % 8 + 8 (L / 8 / T), so
// each head's pooled rows are fetched into one XCD's L2.  Wave (wr, wc) owns the 32 x 32
// sub-tile at (32 wr, 32 wc) as 2 x 2 MFMA tiles.  In MFMA step t the k-slot ks = lane / 16
// carries feature d = ks D/4 + t, so each lane streams a contiguous quarter of its row.
// ---------------------------------------------------------------------------------------
typedef double dbl4 __attribute__((ext_vector_type(4)));

template <int D>
__global__ __launch_bounds__(256) void score_kernel(const double* __restrict__ qbar,
                                                    const double* __restrict__ kbar,
                                                    double* __restrict__ S, double scale,
                                                    int32_t n, int32_t bh, int32_t tiles) {
    constexpr int Q4 = D / 4;
    const uint32_t L = blockIdx.x;
    const uint32_t T = (uint32_t)tiles * tiles;
    const uint32_t k = L >> 3;
    const uint32_t h = (L & 7) + 8 * (k / T);
    if (h >= (uint32_t)bh) return;
    const uint32_t tile = k % T;
    const int ti = tile / tiles, tj = tile - ti * tiles;
    const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
    const int ks = lane >> 4, sub = lane & 15;
    const int row0 = ti * 64 + (w >> 1) * 32;
    const int col0 = tj * 64 + (w & 1) * 32;
    const double* pa[2];
    const double* pb[2];
#pragma unroll
    for (int u = 0; u < 2; ++u) {
        const int r = min(row0 + 16 * u + sub, n - 1);      // rows past n: computed, not stored
        const int c = min(col0 + 16 * u + sub, n - 1);
        pa[u] = qbar + ((size_t)h * n + r) * D + ks * Q4;
        pb[u] = kbar + ((size_t)h * n + c) * D + ks * Q4;
    }
    dbl4 acc[2][2];
#pragma unroll
    for (int u = 0; u < 2; ++u)
#pragma unroll
        for (int v = 0; v < 2; ++v) acc[u][v] = dbl4{0.0, 0.0, 0.0, 0.0};
#pragma unroll 4          // (4: loads of the next steps in flight; 10 % faster routing than 2)
    for (int t0 = 0; t0 < Q4; t0 += 4) {
        double2 av[2][2], bv[2][2];
#pragma unroll
        for (int u = 0; u < 2; ++u) {
            av[u][0] = *(const double2*)(pa[u] + t0);
            av[u][1] = *(const double2*)(pa[u] + t0 + 2);
            bv[u][0] = *(const double2*)(pb[u] + t0);
            bv[u][1] = *(const double2*)(pb[u] + t0 + 2);
        }
#pragma unroll
        for (int st = 0; st < 4; ++st)
#pragma unroll
            for (int u = 0; u < 2; ++u)
#pragma unroll
                for (int v = 0; v < 2; ++v) {
                    const double x = (st & 1) ? av[u][st >> 1].y : av[u][st >> 1].x;
                    const double y = (st & 1) ? bv[v][st >> 1].y : bv[v][st >> 1].x;
                    acc[u][v] = __builtin_amdgcn_mfma_f64_16x16x4f64(x, y, acc[u][v], 0, 0, 0);
                }
    }
    // accumulator element e of a lane holds tile row 4 e + ks, tile column sub
#pragma unroll
    for (int u = 0; u < 2; ++u)
#pragma unroll
        for (int v = 0; v < 2; ++v) {
            const int j = col0 + 16 * v + sub;
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                const int i = row0 + 16 * u + 4 * e + ks;
                if (i < n && j < n) S[((size_t)h * n + i) * n + j] = scale * acc[u][v][e];
            }
        }
}

// ---------------------------------------------------------------------------------------
// route_sort: one wavefront per row (n_blk <= 2048), four rows per workgroup, no barriers.
// Lane l holds sorted positions e = EPL l + r, r < EPL (64 EPL = P2 >= n_blk).  Each block is
// one 64-bit word: the order key of its score (ascending key = descending score) with the
// low log2(P2) bits replaced by the block index, so the words are distinct and ascending
// word order is descending score with ties, down to 2^-(52 - log2 P2) relative, going to the
// smaller index.  Bitonic network: distances below EPL swap registers, the others exchange
// lanes (DPP within a row of 16, permlane swaps across rows and halves).  Then the exact
// scores are gathered in sorted order for the block mass, its prefix, the cut and the bitmap.
// ---------------------------------------------------------------------------------------
constexpr int kSortRows = 4;                   // wavefronts (rows) per workgroup
constexpr int kSortMaxWords = 64;              // bitmap words per row, n_blk <= 2048

struct SortArgs {
    const double* scores;   // [rows][n]
    uint32_t* bitmap;       // [rows][nwords]
    int32_t* counts;        // [rows]
    double top_p;
    int32_t k_floor;
    int32_t n_blk;
    int32_t nwords;
    int64_t rows;
};

// value of lane (l ^ M) for a lane distance M in {1, 2, 4, 8, 16, 32}
template <int M>
__device__ __forceinline__ uint32_t lane_xor(uint32_t v) {
    const int x = (int)v;
    if constexpr (M == 1) {
        return (uint32_t)__builtin_amdgcn_mov_dpp(x, 0xB1, 0xF, 0xF, false);   // quad [1,0,3,2]
    } else if constexpr (M == 2) {
        return (uint32_t)__builtin_amdgcn_mov_dpp(x, 0x4E, 0xF, 0xF, false);   // quad [2,3,0,1]
    } else if constexpr (M == 4) {
        // mirror within 8 lanes (i -> 7 - i), then quad [3,2,1,0] (i -> i ^ 3): i -> i ^ 4
        const int y = __builtin_amdgcn_mov_dpp(x, 0x141, 0xF, 0xF, false);
        return (uint32_t)__builtin_amdgcn_mov_dpp(y, 0x1B, 0xF, 0xF, false);
    } else if constexpr (M == 8) {
        return (uint32_t)__builtin_amdgcn_mov_dpp(x, 0x128, 0xF, 0xF, false);  // rotate row by 8
    } else if constexpr (M == 16) {
        const auto r = __builtin_amdgcn_permlane16_swap(v, v, false, false);
        return (threadIdx.x & 16) ? r[0] : r[1];
    } else {
        const auto r = __builtin_amdgcn_permlane32_swap(v, v, false, false);
        return (threadIdx.x & 32) ? r[0] : r[1];
    }
}

template <int M>
__device__ __forceinline__ uint64_t lane_xor64(uint64_t v) {
    const uint32_t lo = lane_xor<M>((uint32_t)v);
    const uint32_t hi = lane_xor<M>((uint32_t)(v >> 32));
    return ((uint64_t)hi << 32) | lo;
}

// one pass (block size KK, distance JJ) of the ascending bitonic network, then the passes of
// the smaller distances
template <int EPL, int KK, int JJ>
__device__ __forceinline__ void bitonic_passes(uint64_t (&key)[EPL], int lane) {
    if constexpr (JJ < EPL) {
#pragma unroll
        for (int r = 0; r < EPL; ++r) {
            if (r & JJ) continue;
            const int rp = r | JJ;
            const bool up = KK < EPL ? (r & KK) == 0 : (lane & (KK / EPL)) == 0;
            const bool sw = (key[r] > key[rp]) == up;
            const uint64_t a = key[r], b = key[rp];
            key[r] = sw ? b : a;
            key[rp] = sw ? a : b;
        }
    } else {
        constexpr int M = JJ / EPL;
        const bool wmax = ((lane & M) == 0) != ((lane & (KK / EPL)) == 0);
#pragma unroll
        for (int r = 0; r < EPL; ++r) {
            const uint64_t p = lane_xor64<M>(key[r]);
            key[r] = ((key[r] > p) != wmax) ? p : key[r];
        }
    }
    if constexpr (JJ > 1) bitonic_passes<EPL, KK, JJ / 2>(key, lane);
}

template <int EPL, int KK>
__device__ __forceinline__ void bitonic_sort(uint64_t (&key)[EPL], int lane) {
    bitonic_passes<EPL, KK, KK / 2>(key, lane);
    if constexpr (KK < 64 * EPL) bitonic_sort<EPL, 2 * KK>(key, lane);
}

__device__ __forceinline__ double wave_sum(double v) {
#pragma unroll
    for (int m = 32; m > 0; m >>= 1) v += __shfl_xor(v, m, 64);
    return v;
}

template <int EPL>
__global__ __launch_bounds__(kSortRows * 64) void route_sort_kernel(SortArgs a) {
    constexpr int IB = 6 + (EPL >= 2) + (EPL >= 4) + (EPL >= 8) + (EPL >= 16) + (EPL >= 32);
    constexpr uint64_t IM = (1ull << IB) - 1;
    __shared__ uint32_t bits[kSortRows][kSortMaxWords];
    const int lane = threadIdx.x & 63;
    const int w = threadIdx.x >> 6;
    const int64_t row = (int64_t)blockIdx.x * kSortRows + w;
    if (row >= a.rows) return;
    const int n = a.n_blk;
    const double* srow = a.scores + row * n;
    for (int q = lane; q < a.nwords; q += 64) bits[w][q] = 0u;

    uint64_t key[EPL];
#pragma unroll
    for (int r = 0; r < EPL; ++r) {
        const int e = EPL * lane + r;
        key[r] = e < n ? (desc_key(srow[e]) & ~IM) | (uint64_t)e : ~0ull;
    }
    bitonic_sort<EPL, 2>(key, lane);

    // exact scores in sorted order; position 0 (lane 0, r 0) holds the row maximum
    double m[EPL];
#pragma unroll
    for (int r = 0; r < EPL; ++r) {
        const int e = EPL * lane + r;
        m[r] = e < n ? srow[key[r] & IM] : 0.0;
    }
    const uint64_t mb = (uint64_t)__double_as_longlong(m[0]);
    const uint32_t mlo = __builtin_amdgcn_readfirstlane((uint32_t)mb);
    const uint32_t mhi = __builtin_amdgcn_readfirstlane((uint32_t)(mb >> 32));
    const double smax = __longlong_as_double((long long)(((uint64_t)mhi << 32) | mlo));
    double local = 0.0;
#pragma unroll
    for (int r = 0; r < EPL; ++r) {
        const int e = EPL * lane + r;
        m[r] = e < n ? exp(m[r] - smax) : 0.0;
        local += m[r];
    }
    const double Z = wave_sum(local);
    double run = 0.0;
#pragma unroll
    for (int r = 0; r < EPL; ++r) {
        m[r] = m[r] / Z;
        run += m[r];
    }
    // exclusive prefix of the lane totals
    double incl = run;
#pragma unroll
    for (int off = 1; off < 64; off <<= 1) {
        const double u = __shfl_up(incl, off, 64);
        if (lane >= off) incl += u;
    }
    double cum = incl - run;
    int first = n;                                     // first position with cum >= top_p
#pragma unroll
    for (int r = 0; r < EPL; ++r) {
        const int e = EPL * lane + r;
        cum += m[r];
        if (first == n && e < n && cum >= a.top_p) first = e;
    }
#pragma unroll
    for (int off = 32; off > 0; off >>= 1) first = min(first, __shfl_xor(first, off, 64));
    int kp;
    if (a.top_p >= 1.0) kp = n;
    else if (a.top_p <= 0.0) kp = 0;
    else kp = first < n ? first + 1 : n;
    const int c = min(n, max(kp, a.k_floor));
    __builtin_amdgcn_fence(__ATOMIC_SEQ_CST, "wavefront");   // zeroed words, then bit sets
    __builtin_amdgcn_wave_barrier();
#pragma unroll
    for (int r = 0; r < EPL; ++r) {
        const int e = EPL * lane + r;
        const uint32_t j = (uint32_t)(key[r] & IM);
        if (e < c) atomicOr(&bits[w][j >> 5], 1u << (j & 31));
    }
    __builtin_amdgcn_fence(__ATOMIC_SEQ_CST, "wavefront");   // bit sets, then reads
    __builtin_amdgcn_wave_barrier();
    for (int q = lane; q < a.nwords; q += 64) a.bitmap[row * a.nwords + q] = bits[w][q];
    if (lane == 0) a.counts[row] = c;
}

// ---------------------------------------------------------------------------------------
// scan: one workgroup; counts -> row_ptr (exclusive, rows + 1 entries) and nnz
// ---------------------------------------------------------------------------------------
constexpr int kScanThreads = 1024;
constexpr int kScanTile = 4 * kScanThreads;    // counts per pass, four per thread

__global__ __launch_bounds__(kScanThreads) void scan_kernel(const int32_t* __restrict__ counts,
                                                            int32_t* __restrict__ row_ptr,
                                                            int32_t* __restrict__ nnz,
                                                            int64_t rows) {
    __shared__ int32_t wtot[kScanThreads / 64];
    const int t = threadIdx.x;
    const int lane = t & 63, w = t >> 6;
    int32_t carry = 0;                     // total of the earlier passes (nnz fits int32)
    for (int64_t base = 0; base < rows; base += kScanTile) {
        const int64_t i0 = base + 4 * t;
        int32_t v[4];
        if (i0 + 3 < rows) {
            const int4 x = *(const int4*)(counts + i0);      // counts is 256-byte aligned
            v[0] = x.x; v[1] = x.y; v[2] = x.z; v[3] = x.w;
        } else {
#pragma unroll
            for (int u = 0; u < 4; ++u) v[u] = i0 + u < rows ? counts[i0 + u] : 0;
        }
        const int32_t tsum = v[0] + v[1] + v[2] + v[3];
        int32_t incl = tsum;                                 // inclusive over the wavefront
#pragma unroll
        for (int off = 1; off < 64; off <<= 1) {
            const int32_t u = __shfl_up(incl, off, 64);
            if (lane >= off) incl += u;
        }
        if (lane == 63) wtot[w] = incl;
        __syncthreads();
        int32_t before = carry, total = carry;
#pragma unroll
        for (int k = 0; k < kScanThreads / 64; ++k) {
            const int32_t x = wtot[k];
            before += k < w ? x : 0;
            total += x;
        }
        __syncthreads();                                     // wtot is rewritten next pass
        int32_t run = before + incl - tsum;
#pragma unroll
        for (int u = 0; u < 4; ++u) {
            if (i0 + u < rows) row_ptr[i0 + u] = run;
            run += v[u];
        }
        carry = total;
    }
    if (t == 0) {
        row_ptr[rows] = carry;
        nnz[0] = carry;
    }
}

// ---------------------------------------------------------------------------------------
// fill: one wavefront per row; grid (ceil(rows / 4)), 256 threads.  Each half-wavefront expands
// one 32-bit bitmap word per pass, lane b writing column 32 w + b at its rank among the set
// bits, so a pass stores two contiguous runs of ascending columns.
// ---------------------------------------------------------------------------------------
__global__ __launch_bounds__(kThreads) void fill_kernel(const uint32_t* __restrict__ bitmap,
                                                        const int32_t* __restrict__ row_ptr,
                                                        int32_t* __restrict__ col_idx,
                                                        int64_t rows, int32_t nwords) {
    const int lane = threadIdx.x & 63;
    const int64_t row = (int64_t)blockIdx.x * (kThreads / 64) + (threadIdx.x >> 6);
    if (row >= rows) return;
    const uint32_t* bm = bitmap + row * nwords;
    const int bit = lane & 31, hi = lane >> 5;
    int32_t base = row_ptr[row];
    for (int w0 = 0; w0 < nwords; w0 += 2) {
        const int w = w0 + hi;
        const uint32_t word = w < nwords ? bm[w] : 0u;
        const int c0 = __popc(__shfl(word, 0, 64));         // set bits of word w0
        const int c1 = __popc(__shfl(word, 32, 64));        // and of word w0 + 1
        if ((word >> bit) & 1u)
            col_idx[base + (hi ? c0 : 0) + __popc(word & ((1u << bit) - 1u))] = w * 32 + bit;
        base += c0 + c1;
    }
}

// ---------------------------------------------------------------------------------------
// Static periodic-stripe masks (PSA page, "Approach": one six-parameter mask
// M(Tw, To, Ts, Sw, So, Ss) per head, run by the same block-sparse kernel).  Block coordinates
// are those of the tile holding the block's first token: bt = t / tt, bs = (h / th) nW + w / tw.
// Key block j is kept for query block i iff (bt_j - bt_i - To) mod Ts < Tw and
// (bs_j - bs_i - So) mod Ss < Sw (non-negative remainders).  One wavefront per row, four rows
// per workgroup; 64 key blocks per ballot give two bitmap words.  The coordinates of every
// block are computed once per call (`coord_kernel`) into the workspace.
// ---------------------------------------------------------------------------------------
struct StripeArgs {
    const int32_t* params;  // [heads][6] = Tw, To, Ts, Sw, So, Ss
    int2* coords;           // [n_blk] (bt, bs)
    uint32_t* bitmap;       // [rows][nwords]
    int32_t* counts;        // [rows]
    GridArgs g;
    int32_t B, n_blk, heads, nwords;
    int64_t rows;
};

__device__ __forceinline__ void block_coord(int32_t j, const StripeArgs& a, int32_t& bt,
                                            int32_t& bs) {
    const uint32_t n = tile_pos_to_raster((uint32_t)j * (uint32_t)a.B, a.g);
    const uint32_t HW = (uint32_t)a.g.H * (uint32_t)a.g.W;
    const uint32_t t = n / HW;
    const uint32_t r = n - t * HW;
    const uint32_t h = r / (uint32_t)a.g.W;
    const uint32_t w = r - h * (uint32_t)a.g.W;
    const int32_t nW = (a.g.W + a.g.tw - 1) / a.g.tw;
    bt = (int32_t)(t / (uint32_t)a.g.tt);
    bs = (int32_t)(h / (uint32_t)a.g.th) * nW + (int32_t)(w / (uint32_t)a.g.tw);
}

__global__ __launch_bounds__(kThreads) void coord_kernel(StripeArgs a) {
    const int32_t j = blockIdx.x * kThreads + threadIdx.x;
    if (j >= a.n_blk) return;
    int32_t bt, bs;
    block_coord(j, a, bt, bs);
    a.coords[j] = make_int2(bt, bs);
}

__device__ __forceinline__ int32_t nonneg_mod(int32_t x, int32_t m) {
    const int32_t r = x % m;
    return r < 0 ? r + m : r;
}

__global__ __launch_bounds__(kThreads) void stripe_kernel(StripeArgs a) {
    const int lane = threadIdx.x & 63;
    const int64_t row = (int64_t)blockIdx.x * (kThreads / 64) + (threadIdx.x >> 6);
    if (row >= a.rows) return;
    const int32_t n = a.n_blk;
    const int64_t bh = row / n;
    const int32_t i = (int32_t)(row - bh * n);
    const int32_t* p = a.params + 6 * (int32_t)(bh % a.heads);
    const int32_t Tw = p[0], To = p[1], Ts = p[2], Sw = p[3], So = p[4], Ss = p[5];
    const int2 ci = a.coords[i];
    int32_t count = 0;
    for (int32_t j0 = 0; j0 < n; j0 += 64) {
        const int32_t j = j0 + lane;
        bool keep = false;
        if (j < n) {
            const int2 cj = a.coords[j];
            keep = nonneg_mod(cj.x - ci.x - To, Ts) < Tw && nonneg_mod(cj.y - ci.y - So, Ss) < Sw;
        }
        const uint64_t m = __ballot(keep);
        count += __popcll(m);
        const int32_t w0 = j0 >> 5;
        if (lane == 0) a.bitmap[row * a.nwords + w0] = (uint32_t)m;
        if (lane == 1 && w0 + 1 < a.nwords) a.bitmap[row * a.nwords + w0 + 1] = (uint32_t)(m >> 32);
    }
    if (lane == 0) a.counts[row] = count;
}

struct RouteLayout {
    size_t qbar, kbar, bitmap, counts, scores, total;
};

RouteLayout route_layout(int32_t batch, int32_t heads, int32_t D, const Geometry& g) {
    RouteLayout L;
    const size_t bh = (size_t)batch * heads;
    const size_t rows = bh * g.n_blk;
    const size_t nwords = (g.n_blk + 31) / 32;
    size_t off = 0;
    L.qbar = off;   off = align_up(off + bh * g.n_blk * D * 8, 256);
    L.kbar = off;   off = align_up(off + bh * g.n_blk * D * 8, 256);
    L.bitmap = off; off = align_up(off + rows * nwords * 4, 256);
    L.counts = off; off = align_up(off + rows * 4, 256);
    L.scores = off;
    if (g.n_blk <= kSortMaxWords * 32) off = align_up(off + rows * (size_t)g.n_blk * 8, 256);
    L.total = off;
    return L;
}

}  // namespace

size_t route_ws_bytes(int32_t batch, int32_t heads, int32_t D, const Geometry& g) {
    return route_layout(batch, heads, D, g).total;
}

bsa_status launch_route(const void* q_t, const void* k_t, int32_t batch, int32_t heads,
                        int32_t D, const Geometry& g, double top_p, int32_t k_floor,
                        double scale, int32_t* row_ptr, int32_t* col_idx, int32_t* nnz,
                        double* block_scores, void* ws, hipStream_t s) {
    const RouteLayout L = route_layout(batch, heads, D, g);
    unsigned char* w = (unsigned char*)ws;
    double* qbar = (double*)(w + L.qbar);
    double* kbar = (double*)(w + L.kbar);
    const int32_t bh = batch * heads;
    dim3 pgrid(g.n_blk, bh, 2);
    if (D == 64)
        hipLaunchKernelGGL(pool_kernel<64>, pgrid, dim3(kThreads), 0, s, (const uint4*)q_t,
                           (const uint4*)k_t, qbar, kbar, g.N, g.Npad, g.B, g.n_blk);
    else
        hipLaunchKernelGGL(pool_kernel<128>, pgrid, dim3(kThreads), 0, s, (const uint4*)q_t,
                           (const uint4*)k_t, qbar, kbar, g.N, g.Npad, g.B, g.n_blk);
    bsa_status st = check_launch("pool");
    if (st != BSA_OK) return st;
    return launch_route_pooled(qbar, kbar, batch, heads, D, g, top_p, k_floor, scale, row_ptr,
                               col_idx, nnz, block_scores, ws, s);
}

bsa_status launch_route_pooled(const double* qbar, const double* kbar, int32_t batch,
                               int32_t heads, int32_t D, const Geometry& g, double top_p,
                               int32_t k_floor, double scale, int32_t* row_ptr,
                               int32_t* col_idx, int32_t* nnz, double* block_scores, void* ws,
                               hipStream_t s) {
    const RouteLayout L = route_layout(batch, heads, D, g);
    unsigned char* w = (unsigned char*)ws;
    uint32_t* bitmap = (uint32_t*)(w + L.bitmap);
    int32_t* counts = (int32_t*)(w + L.counts);
    const int32_t bh = batch * heads;
    const int64_t rows = (int64_t)bh * g.n_blk;
    bsa_status st;

    RouteArgs a;
    a.qbar = qbar;
    a.kbar = kbar;
    a.bitmap = bitmap;
    a.counts = counts;
    a.scores_out = block_scores;
    a.scale = scale;
    a.top_p = top_p;
    a.k_floor = k_floor;
    a.n_blk = g.n_blk;
    int P2 = 1;
    while (P2 < g.n_blk) P2 <<= 1;
    if (P2 < 32) P2 = 32;
    a.P2 = P2;
    int R = (int)(65536 / ((size_t)P2 * 8));
    R = R < 1 ? 1 : (R > 8 ? 8 : R);
    a.R = R;
    a.nwords = (g.n_blk + 31) / 32;
    if (g.n_blk <= kSortMaxWords * 32) {
        // scores by MFMA into block_scores (or the workspace), then one wavefront per row
        double* S = block_scores ? block_scores : (double*)(w + L.scores);
        const int tiles = (g.n_blk + 63) / 64;
        const unsigned sgrid = 8u * (unsigned)(tiles * tiles) * (unsigned)((bh + 7) / 8);
        if (D == 64)
            hipLaunchKernelGGL(score_kernel<64>, dim3(sgrid), dim3(256), 0, s, qbar, kbar, S,
                               scale, g.n_blk, bh, tiles);
        else
            hipLaunchKernelGGL(score_kernel<128>, dim3(sgrid), dim3(256), 0, s, qbar, kbar, S,
                               scale, g.n_blk, bh, tiles);
        st = check_launch("score");
        if (st != BSA_OK) return st;
        SortArgs sa;
        sa.scores = S;
        sa.bitmap = bitmap;
        sa.counts = counts;
        sa.top_p = top_p;
        sa.k_floor = k_floor;
        sa.n_blk = g.n_blk;
        sa.nwords = a.nwords;
        sa.rows = rows;
        const dim3 ogrid((unsigned)((rows + kSortRows - 1) / kSortRows));
        const dim3 oblk(kSortRows * 64);
        const int epl = P2 <= 64 ? 1 : P2 / 64;
        switch (epl) {
            case 1:  hipLaunchKernelGGL(route_sort_kernel<1>, ogrid, oblk, 0, s, sa); break;
            case 2:  hipLaunchKernelGGL(route_sort_kernel<2>, ogrid, oblk, 0, s, sa); break;
            case 4:  hipLaunchKernelGGL(route_sort_kernel<4>, ogrid, oblk, 0, s, sa); break;
            case 8:  hipLaunchKernelGGL(route_sort_kernel<8>, ogrid, oblk, 0, s, sa); break;
            case 16: hipLaunchKernelGGL(route_sort_kernel<16>, ogrid, oblk, 0, s, sa); break;
            default: hipLaunchKernelGGL(route_sort_kernel<32>, ogrid, oblk, 0, s, sa); break;
        }
    } else {
        // longer rows: one workgroup scores and sorts R rows in LDS
        const size_t lds = route_lds_bytes(D, a.P2, R) + 16;
        dim3 rgrid((g.n_blk + R - 1) / R, bh);
        if (D == 64) {
            (void)hipFuncSetAttribute((const void*)route_kernel<64>,
                                hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
            hipLaunchKernelGGL(route_kernel<64>, rgrid, dim3(kThreads), lds, s, a);
        } else {
            (void)hipFuncSetAttribute((const void*)route_kernel<128>,
                                hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
            hipLaunchKernelGGL(route_kernel<128>, rgrid, dim3(kThreads), lds, s, a);
        }
    }
    st = check_launch("route");
    if (st != BSA_OK) return st;

    hipLaunchKernelGGL(scan_kernel, dim3(1), dim3(kScanThreads), 0, s, counts, row_ptr, nnz,
                       rows);
    st = check_launch("scan");
    if (st != BSA_OK) return st;

    hipLaunchKernelGGL(fill_kernel, dim3((unsigned)((rows + 3) / 4)), dim3(kThreads), 0, s,
                       bitmap, row_ptr, col_idx, rows, a.nwords);
    return check_launch("fill");
}

size_t stripe_ws_bytes(int32_t batch, int32_t heads, const Geometry& g) {
    const size_t rows = (size_t)batch * heads * g.n_blk;
    const size_t nwords = (g.n_blk + 31) / 32;
    return align_up(rows * nwords * 4, 256) + align_up(rows * 4, 256) +
           align_up((size_t)heads * 6 * 4, 256) + align_up((size_t)g.n_blk * 8, 256);
}

bsa_status launch_stripe(const int32_t* params_host, int32_t batch, int32_t heads,
                         const Geometry& g, int32_t* row_ptr, int32_t* col_idx, int32_t* nnz,
                         void* ws, hipStream_t s) {
    const int64_t rows = (int64_t)batch * heads * g.n_blk;
    const int32_t nwords = (g.n_blk + 31) / 32;
    unsigned char* w = (unsigned char*)ws;
    StripeArgs a;
    a.bitmap = (uint32_t*)w;
    a.counts = (int32_t*)(w + align_up((size_t)rows * nwords * 4, 256));
    int32_t* params = (int32_t*)(w + align_up((size_t)rows * nwords * 4, 256) +
                                 align_up((size_t)rows * 4, 256));
    a.coords = (int2*)((unsigned char*)params + align_up((size_t)heads * 6 * 4, 256));
    if (hipMemcpyAsync(params, params_host, (size_t)heads * 6 * 4, hipMemcpyHostToDevice, s) !=
        hipSuccess)
        return fail(BSA_ERR_HIP, "stripe parameters: copy to the workspace failed");
    a.params = params;
    a.g = GridArgs{g.T, g.H, g.W, g.tt, g.th, g.tw, g.order};
    a.B = g.B;
    a.n_blk = g.n_blk;
    a.heads = heads;
    a.nwords = nwords;
    a.rows = rows;
    hipLaunchKernelGGL(coord_kernel, dim3((unsigned)((g.n_blk + kThreads - 1) / kThreads)),
                       dim3(kThreads), 0, s, a);
    bsa_status st = check_launch("stripe coordinates");
    if (st != BSA_OK) return st;
    hipLaunchKernelGGL(stripe_kernel, dim3((unsigned)((rows + 3) / 4)), dim3(kThreads), 0, s, a);
    st = check_launch("stripe");
    if (st != BSA_OK) return st;
    hipLaunchKernelGGL(scan_kernel, dim3(1), dim3(kScanThreads), 0, s, a.counts, row_ptr, nnz,
                       rows);
    st = check_launch("scan");
    if (st != BSA_OK) return st;
    hipLaunchKernelGGL(fill_kernel, dim3((unsigned)((rows + 3) / 4)), dim3(kThreads), 0, s,
                       a.bitmap, row_ptr, col_idx, rows, nwords);
    return check_launch("fill");
}

bsa_status launch_scan(const int32_t* counts, int32_t* excl, int32_t* total, int64_t n,
                       hipStream_t s) {
    hipLaunchKernelGGL(scan_kernel, dim3(1), dim3(kScanThreads), 0, s, counts, excl, total, n);
    return check_launch("scan");
}

}  // namespace bsa
