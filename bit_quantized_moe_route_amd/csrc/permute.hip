// Token permutation: a stable counting sort of the T*k assignments by expert,
// and the fused route + permute kernel for decode batches.
//
// Batches up to T*k = 4096, one workgroup of 1024 threads:
//   1. histogram of expert ids in LDS;
//   2. exclusive prefix scan over the E counts (wave scans + a scan of the
//      wave totals) -> counts, offsets;
//   3. the assignments in chunks of 1024, in order: within a wave, lanes
//      with the same expert find each other with 11 ballots (one per bit
//      of the id); a lane's rank is its position among its peers, plus the
//      peers in earlier waves of the chunk (per-wave counts in LDS), plus
//      the running count of that expert from earlier chunks.
// Large batches split the assignments into B <= 64 contiguous slices, one
// workgroup each, in two launches:
//   1. each workgroup writes its slice's histogram to the workspace [B][E];
//   2. each workgroup sums the histograms (all of them for the offsets,
//      those of earlier slices for its own starting slot per expert) and
//      ranks and scatters its slice as in step 3 above.
// Decode batches (T*k <= 64) route and sort in one launch of one workgroup
// (see k_route_permute_small).  Either way the result is unique, so it does
// not depend on timing.
#include "topk_dev.h"

namespace moeq {

namespace {

constexpr int kPermThreads = 1024;
constexpr int kPermWaves = kPermThreads / 64;
__host__ __device__ constexpr size_t permute_lds_bytes(int E) {
    return (size_t)(2 * E + kPermWaves) * sizeof(int) + (size_t)kPermWaves * E;
}

// Exclusive scan over the workgroup of c (threads tid < E hold the values,
// E <= kPermThreads); returns the thread's exclusive prefix.  wtot: LDS
// [kPermWaves].  Ends with a barrier.
__device__ __forceinline__ int block_exclusive_scan(int c, int* wtot) {
    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = tid >> 6;
    int incl = c;
#pragma unroll
    for (int off = 1; off < 64; off <<= 1) {
        int o = __shfl_up(incl, off);
        if (lane >= off) incl += o;
    }
    if (lane == 63) wtot[wave] = incl;
    __syncthreads();
    int wbase = 0;
    for (int w = 0; w < wave; ++w) wbase += wtot[w];
    __syncthreads();
    return wbase + incl - c;
}

// Ranks the assignments a0 .. a1-1 in order and scatters them: run[e] is the
// next free slot of expert e (LDS, advanced here); wcnt: LDS
// [kPermWaves][E] bytes, zero on entry and on exit.
__device__ __forceinline__ void rank_scatter(const int32_t* ids, int a0, int a1, int E, int* run,
                                             uint8_t* wcnt, int32_t* __restrict__ perm_src,
                                             int32_t* __restrict__ inv_perm) {
    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = tid >> 6;
    const uint64_t lt_mask = (lane == 0) ? 0ull : (~0ull >> (64 - lane));
    for (int base = a0; base < a1; base += kPermThreads) {
        const int a = base + tid;
        const bool valid = a < a1;
        const int e = valid ? ids[a] : 0x7ff;   // sentinel never equals an id
        uint64_t peers = ~0ull;
#pragma unroll
        for (int b = 0; b < 11; ++b) {
            uint64_t bal = __ballot((e >> b) & 1);
            peers &= ((e >> b) & 1) ? bal : ~bal;
        }
        const int rank_w = __popcll(peers & lt_mask);
        if (valid && rank_w == 0) wcnt[wave * E + e] = (uint8_t)__popcll(peers);
        __syncthreads();
        if (valid) {
            int r = run[e] + rank_w;
            for (int w = 0; w < wave; ++w) r += wcnt[w * E + e];
            perm_src[r] = a;
            inv_perm[a] = r;
        }
        __syncthreads();
        for (int x = tid; x < E; x += kPermThreads) {
            int s = 0;
            for (int w = 0; w < kPermWaves; ++w) {
                s += wcnt[w * E + x];
                wcnt[w * E + x] = 0;
            }
            run[x] += s;
        }
        __syncthreads();
    }
}

// The whole sort in one workgroup.  ids may point to global memory or to LDS.
__device__ __forceinline__ void permute_body(const int32_t* ids, int n, int E,
                                             int32_t* __restrict__ counts,
                                             int32_t* __restrict__ offsets,
                                             int32_t* __restrict__ perm_src,
                                             int32_t* __restrict__ inv_perm, int* smem) {
    int* hist = smem;                 // [E]
    int* run = smem + E;              // [E]
    int* wtot = smem + 2 * E;         // [kPermWaves]
    uint8_t* wcnt = reinterpret_cast<uint8_t*>(smem + 2 * E + kPermWaves);  // [kPermWaves][E]
    const int tid = threadIdx.x;

    for (int e = tid; e < E; e += kPermThreads) hist[e] = 0;
    for (int i = tid; i < kPermWaves * E; i += kPermThreads) wcnt[i] = 0;
    __syncthreads();
    for (int a = tid; a < n; a += kPermThreads) atomicAdd(&hist[ids[a]], 1);
    __syncthreads();

    const int c = tid < E ? hist[tid] : 0;
    const int excl = block_exclusive_scan(c, wtot);
    if (tid < E) {
        counts[tid] = c;
        offsets[tid] = excl;
        run[tid] = excl;
    }
    if (tid == 0) offsets[E] = n;
    __syncthreads();
    rank_scatter(ids, 0, n, E, run, wcnt, perm_src, inv_perm);
}

// Large batches, launch 1: the histogram of slice blockIdx.x
// (assignments slice*C .. min(n, slice*C + C)) -> hist_ws[slice][E].
__global__ __launch_bounds__(kPermThreads) void k_perm_hist(const int32_t* __restrict__ ids, int n,
                                                            int E, int C,
                                                            int32_t* __restrict__ hist_ws) {
    extern __shared__ int smem[];
    const int tid = threadIdx.x;
    for (int e = tid; e < E; e += kPermThreads) smem[e] = 0;
    __syncthreads();
    const int a0 = blockIdx.x * C;
    const int a1 = min(n, a0 + C);
    for (int a = a0 + tid; a < a1; a += kPermThreads) atomicAdd(&smem[ids[a]], 1);
    __syncthreads();
    for (int e = tid; e < E; e += kPermThreads) hist_ws[(int64_t)blockIdx.x * E + e] = smem[e];
}

// Large batches, launch 2: offsets from the nb slice histograms, then slice
// blockIdx.x ranked and scattered from its own starting slots.
__global__ __launch_bounds__(kPermThreads) void k_perm_scatter(
    const int32_t* __restrict__ ids, int n, int E, int C, int nb,
    const int32_t* __restrict__ hist_ws, int32_t* __restrict__ counts,
    int32_t* __restrict__ offsets, int32_t* __restrict__ perm_src,
    int32_t* __restrict__ inv_perm) {
    extern __shared__ int smem[];
    int* run = smem;                  // [E]
    int* wtot = smem + E;             // [kPermWaves]
    uint8_t* wcnt = reinterpret_cast<uint8_t*>(smem + E + kPermWaves);  // [kPermWaves][E]
    const int tid = threadIdx.x;
    const int slice = blockIdx.x;
    for (int i = tid; i < kPermWaves * E; i += kPermThreads) wcnt[i] = 0;
    int total = 0, before = 0;
    if (tid < E) {
        for (int b = 0; b < nb; ++b) {
            const int v = hist_ws[(int64_t)b * E + tid];
            total += v;
            before += b < slice ? v : 0;
        }
    }
    const int excl = block_exclusive_scan(total, wtot);
    if (tid < E) {
        run[tid] = excl + before;
        if (slice == 0) {
            counts[tid] = total;
            offsets[tid] = excl;
        }
    }
    if (slice == 0 && tid == 0) offsets[E] = n;
    __syncthreads();
    const int a0 = slice * C;
    rank_scatter(ids, a0, min(n, a0 + C), E, run, wcnt, perm_src, inv_perm);
}

__global__ __launch_bounds__(kPermThreads) void k_permute(const int32_t* __restrict__ ids,
                                                          int n, int E,
                                                          int32_t* __restrict__ counts,
                                                          int32_t* __restrict__ offsets,
                                                          int32_t* __restrict__ perm_src,
                                                          int32_t* __restrict__ inv_perm) {
    extern __shared__ int smem[];
    permute_body(ids, n, E, counts, offsets, perm_src, inv_perm, smem);
}

// Route + permute for T*k <= 64 (decode): one workgroup of min(T, 16)
// waves routes the tokens (ids also to LDS); wave 0 then sorts the n = T*k
// assignments, lane a holding assignment a: an LDS histogram, a wave scan of
// the E counts (lane L sums experts L*per .. L*per + per - 1), and the rank
// of a among the lanes with the same expert (11 ballots) added to that
// expert's offset.
constexpr int kSmallAssign = 64;
constexpr int kSmallMaxWaves = 16;

template <int VPL>
__global__ __launch_bounds__(64 * kSmallMaxWaves) void k_route_permute_small(
    const float* __restrict__ logits, int T, int E, int k, int32_t* __restrict__ ids,
    float* __restrict__ w, int32_t* __restrict__ counts, int32_t* __restrict__ offsets,
    int32_t* __restrict__ perm_src, int32_t* __restrict__ inv_perm) {
    __shared__ int sids[kSmallAssign];
    __shared__ int hist[MOE_MAX_E];
    const int lane = threadIdx.x & 63;
    const int wave = threadIdx.x >> 6;
    const int nw = blockDim.x >> 6;
    for (int x = threadIdx.x; x < E; x += blockDim.x) hist[x] = 0;
    for (int t = wave; t < T; t += nw)
        route_token<VPL>(logits + (int64_t)t * E, E, k, lane, ids + (int64_t)t * k,
                         w + (int64_t)t * k, sids + t * k);
    __syncthreads();
    const int n = T * k;
    const bool valid = lane < n;
    const int e = valid ? sids[lane] : 0x7ff;   // sentinel never equals an id
    if (wave == 0 && valid) atomicAdd(&hist[e], 1);
    __syncthreads();
    if (wave != 0) return;
    // exclusive scan of hist over the experts: lane L owns a run of `per`
    const int per = (E + 63) / 64;
    const int e0 = lane * per;
    int sum = 0;
    for (int i = 0; i < per; ++i)
        if (e0 + i < E) sum += hist[e0 + i];
    int incl = sum;
#pragma unroll
    for (int off = 1; off < 64; off <<= 1) {
        const int v = __shfl_up(incl, off);
        if (lane >= off) incl += v;
    }
    int run = incl - sum;
    for (int i = 0; i < per; ++i) {
        const int x = e0 + i;
        if (x < E) {
            const int c = hist[x];
            counts[x] = c;
            offsets[x] = run;
            hist[x] = run;   // this expert's first slot, for the ranks below
            run += c;
        }
    }
    if (lane == 0) offsets[E] = n;
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "workgroup");
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "workgroup");
    uint64_t peers = ~0ull;
#pragma unroll
    for (int b = 0; b < 11; ++b) {
        const uint64_t bal = __ballot((e >> b) & 1);
        peers &= ((e >> b) & 1) ? bal : ~bal;
    }
    const uint64_t lt_mask = (lane == 0) ? 0ull : (~0ull >> (64 - lane));
    if (valid) {
        const int r = hist[e] + __popcll(peers & lt_mask);
        perm_src[r] = lane;
        inv_perm[lane] = r;
    }
}

}  // namespace

// Slices of the large-batch path: at least kPermSlice assignments each, at
// most kPermMaxSlices of them.
constexpr int kPermSlice = 2048;
constexpr int kPermMaxSlices = 64;

// one-workgroup permute up to this many assignments
constexpr int kSingleMaxAssign = 4096;

bool permute_single(int64_t n) { return n <= kSingleMaxAssign; }

int permute_slice(int64_t n) {
    int64_t c = (n + kPermMaxSlices - 1) / kPermMaxSlices;
    c = (c + kPermThreads - 1) / kPermThreads * kPermThreads;
    return (int)(c < kPermSlice ? kPermSlice : c);
}

size_t permute_ws_bytes(int64_t T, int32_t k, int32_t E) {
    const int64_t n = T * k;
    if (permute_single(n)) return 0;
    const int64_t nb = (n + permute_slice(n) - 1) / permute_slice(n);
    return (size_t)(nb * E) * sizeof(int32_t);
}

int launch_permute(const int32_t* ids, int64_t T, int32_t k, int32_t E, int32_t* counts,
                   int32_t* offsets, int32_t* perm_src, int32_t* inv_perm, void* ws,
                   void* stream) {
    hipStream_t s = reinterpret_cast<hipStream_t>(stream);
    const int n = (int)(T * k);
    if (permute_single(n)) {
        k_permute<<<1, kPermThreads, permute_lds_bytes(E), s>>>(ids, n, E, counts, offsets,
                                                                perm_src, inv_perm);
        MOEQ_CHECK_LAUNCH();
        return MOE_OK;
    }
    const int C = permute_slice(n);
    const int nb = (n + C - 1) / C;
    int32_t* hist = static_cast<int32_t*>(ws);
    k_perm_hist<<<nb, kPermThreads, (size_t)E * sizeof(int), s>>>(ids, n, E, C, hist);
    MOEQ_CHECK_LAUNCH();
    const size_t lds = (size_t)(E + kPermWaves) * sizeof(int) + (size_t)kPermWaves * E;
    k_perm_scatter<<<nb, kPermThreads, lds, s>>>(ids, n, E, C, nb, hist, counts, offsets,
                                                 perm_src, inv_perm);
    MOEQ_CHECK_LAUNCH();
    return MOE_OK;
}

bool route_permute_fused_ok(int64_t T, int32_t k) { return T * k <= kSmallAssign; }

int launch_route_permute(const float* logits, int64_t T, int32_t E, int32_t k, int32_t* ids,
                         float* w, int32_t* counts, int32_t* offsets, int32_t* perm_src,
                         int32_t* inv_perm, void* stream) {
    hipStream_t s = reinterpret_cast<hipStream_t>(stream);
    const int waves = T < kSmallMaxWaves ? (int)T : kSmallMaxWaves;
    const int nt = 64 * (waves > 0 ? waves : 1);
    if (E <= 256)
        k_route_permute_small<4><<<1, nt, 0, s>>>(logits, (int)T, E, k, ids, w, counts, offsets,
                                                 perm_src, inv_perm);
    else
        k_route_permute_small<16><<<1, nt, 0, s>>>(logits, (int)T, E, k, ids, w, counts, offsets,
                                                  perm_src, inv_perm);
    MOEQ_CHECK_LAUNCH();
    return MOE_OK;
}

}  // namespace moeq
