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
// scan: one workgroup; counts -> row_ptr (exclusive, rows + 1 entries) and nnz
// ---------------------------------------------------------------------------------------
constexpr int kScanThreads = 1024;

__global__ __launch_bounds__(kScanThreads) void scan_kernel(const int32_t* __restrict__ counts,
                                                            int32_t* __restrict__ row_ptr,
                                                            int32_t* __restrict__ nnz,
                                                            int64_t rows) {
    __shared__ int64_t part[kScanThreads];
    const int t = threadIdx.x;
    const int64_t seg = (rows + kScanThreads - 1) / kScanThreads;
    const int64_t lo = min(rows, t * seg), hi = min(rows, lo + seg);
    int64_t local = 0;
    for (int64_t r = lo; r < hi; ++r) local += counts[r];
    part[t] = local;
    __syncthreads();
    for (int off = 1; off < kScanThreads; off <<= 1) {
        const int64_t add = t >= off ? part[t - off] : 0;
        __syncthreads();
        part[t] += add;
        __syncthreads();
    }
    int64_t run = part[t] - local;
    for (int64_t r = lo; r < hi; ++r) {
        row_ptr[r] = (int32_t)run;
        run += counts[r];
    }
    if (t == kScanThreads - 1) {
        row_ptr[rows] = (int32_t)part[t];
        nnz[0] = (int32_t)part[t];
    }
}

// ---------------------------------------------------------------------------------------
// fill: one wavefront per row; grid (ceil(rows / 4)), 256 threads
// ---------------------------------------------------------------------------------------
__global__ __launch_bounds__(kThreads) void fill_kernel(const uint32_t* __restrict__ bitmap,
                                                        const int32_t* __restrict__ row_ptr,
                                                        int32_t* __restrict__ col_idx,
                                                        int64_t rows, int32_t nwords) {
    const int lane = threadIdx.x & 63;
    const int64_t row = (int64_t)blockIdx.x * (kThreads / 64) + (threadIdx.x >> 6);
    if (row >= rows) return;
    const uint32_t* bm = bitmap + row * nwords;
    int32_t base = row_ptr[row];
    for (int w0 = 0; w0 < nwords; w0 += 64) {
        const int w = w0 + lane;
        const uint32_t word = w < nwords ? bm[w] : 0u;
        const int cnt = __popc(word);
        int incl = cnt;
        for (int off = 1; off < 64; off <<= 1) {
            const int up = __shfl_up(incl, off, 64);
            if (lane >= off) incl += up;
        }
        int pos = base + incl - cnt;
        uint32_t m = word;
        while (m) {
            const int bit = __ffs(m) - 1;
            col_idx[pos++] = w * 32 + bit;
            m &= m - 1;
        }
        base += __shfl(incl, 63, 64);
    }
}

struct RouteLayout {
    size_t qbar, kbar, bitmap, counts, total;
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
    uint32_t* bitmap = (uint32_t*)(w + L.bitmap);
    int32_t* counts = (int32_t*)(w + L.counts);
    const int32_t bh = batch * heads;
    const int64_t rows = (int64_t)bh * g.n_blk;

    dim3 pgrid(g.n_blk, bh, 2);
    if (D == 64)
        hipLaunchKernelGGL(pool_kernel<64>, pgrid, dim3(kThreads), 0, s, (const uint4*)q_t,
                           (const uint4*)k_t, qbar, kbar, g.N, g.Npad, g.B, g.n_blk);
    else
        hipLaunchKernelGGL(pool_kernel<128>, pgrid, dim3(kThreads), 0, s, (const uint4*)q_t,
                           (const uint4*)k_t, qbar, kbar, g.N, g.Npad, g.B, g.n_blk);
    bsa_status st = check_launch("pool");
    if (st != BSA_OK) return st;

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
    const size_t lds = route_lds_bytes(D, P2, R) + 16;
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

}  // namespace bsa
