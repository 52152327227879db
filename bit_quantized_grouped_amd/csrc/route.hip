// GPU-resident routing: top-k + softmax weights, expert histogram, exclusive
// prefix scan, stable scatter and the row-block map, with no host round trip
// ([P1] dothoosh.com Lily article, "Prefill optimizations", GPU-resident
// routing bullet; [P1] "Model specification": 256 experts, 8 selected).
//
// Two phases, each a device function:
//   topk_token   one wave per token.  Logits become order-preserving
//                integer keys; a radix select over the key bits (ballot +
//                popcount per bit, stopping as soon as exactly k keys lie
//                at or above the running threshold) finds the k-th largest
//                value; ties at that value go to the lowest expert indices.
//                The k chosen are ranked (value descending, index
//                ascending) through LDS, and their softmax weights formed.
//   group_all    one workgroup of 16 waves over the T*k assignments, cut
//                into 16 contiguous segments.  Pass 1: per-segment expert
//                histograms (ballot match of equal experts inside 64-lane
//                chunks, one LDS update per distinct expert).  Then per
//                expert: prefix over segments, totals (counts), exclusive
//                scan (offsets) and the block map with n_blocks.  Pass 2
//                re-walks the segments; each assignment's row is its
//                segment's base for its expert plus its rank among equal
//                experts earlier in the chunk: a stable counting sort.
// Large T: a top-k kernel with one wave per token, then a one-workgroup
// grouping kernel.  Small T: both phases in one workgroup (one launch).
// Every output is a deterministic function of the logits.
#include "moe_device.h"
#include "moe_launch.h"
#include "moe_topk.h"

namespace moeq4 {

constexpr int kTopkWaves = 4;          // tokens per workgroup in the top-k kernel
constexpr int kGroupThreads = 1024;    // one grouping workgroup: 16 waves
constexpr int kGroupWaves = kGroupThreads / WAVE;
constexpr int kFusedMaxTokens = 64;    // T at or below this: one fused launch

template <int EPL>
__global__ __launch_bounds__(kTopkWaves * WAVE) void route_topk_kernel(
    const float* __restrict__ logits, int T, int E, int k, int32_t* __restrict__ topk_idx,
    float* __restrict__ topk_w) {
    extern __shared__ uint32_t smem_u[];
    const int wave = threadIdx.x / WAVE;
    const int t = blockIdx.x * kTopkWaves + wave;
    uint32_t* s_key = smem_u + wave * 3 * k;
    int* s_e = (int*)(s_key + k);
    float* s_v = (float*)(s_key + 2 * k);
    if (t < T)
        topk_token<EPL>(logits + (size_t)t * E, E, k, topk_idx + (size_t)t * k,
                        topk_w + (size_t)t * k, s_key, s_e, s_v);
}

// Expert of each assignment inside a 64-lane chunk -> (rank among equal
// experts in lower lanes, number of equal experts in the chunk).
__device__ __forceinline__ void match_rank(int e, bool valid, int nbits, int* rank, int* cnt) {
    uint64_t match = __ballot(valid);
    for (int bit = 0; bit < nbits; ++bit) {
        const bool set = (e >> bit) & 1;
        const uint64_t bal = __ballot(valid && set);
        match &= set ? bal : ~bal;
    }
    *rank = __popcll(match & lanemask_lt());
    *cnt = __popcll(match);
}

// Exclusive scan of one value per thread over a kGroupThreads workgroup.
__device__ int block_exclusive_scan(int v, int* s_wave, int* total) {
    const int tid = threadIdx.x, lane = tid % WAVE, wave = tid / WAVE;
    int incl = v;
#pragma unroll
    for (int off = 1; off < WAVE; off <<= 1) {
        const int o = __shfl_up(incl, off, WAVE);
        if (lane >= off) incl += o;
    }
    if (lane == WAVE - 1) s_wave[wave] = incl;
    __syncthreads();
    if (wave == 0) {
        int w = lane < kGroupWaves ? s_wave[lane] : 0;
        int wi = w;
#pragma unroll
        for (int off = 1; off < WAVE; off <<= 1) {
            const int o = __shfl_up(wi, off, WAVE);
            if (lane >= off) wi += o;
        }
        if (lane < kGroupWaves) s_wave[lane] = wi - w;
        if (lane == kGroupWaves - 1) s_wave[kGroupWaves] = wi;
    }
    __syncthreads();
    const int res = s_wave[wave] + incl - v;
    *total = s_wave[kGroupWaves];
    __syncthreads();
    return res;
}

// Histogram, scan, block map and stable scatter of n = T*k assignments
// whose experts are eids[0..n).  Needs kGroupThreads threads and
// kGroupWaves*E + kGroupWaves + 1 ints of LDS at s_hist.
__device__ void group_all(const int32_t* eids, int n, int E, int block_rows, int max_blocks,
                          const RoutingDev& r, int* s_hist) {
    const int tid = threadIdx.x, lane = tid % WAVE, wave = tid / WAVE;
    int* s_wave = s_hist + kGroupWaves * E;
    const int nbits = E > 1 ? 32 - __builtin_clz((unsigned)(E - 1)) : 0;
    const int seg = (n + kGroupWaves - 1) / kGroupWaves;
    const int a_begin = min(n, wave * seg), a_end = min(n, a_begin + seg);
    int* my_hist = s_hist + wave * E;

    for (int i = tid; i < kGroupWaves * E; i += kGroupThreads) s_hist[i] = 0;
    __syncthreads();

    // pass 1: per-segment histograms.  The segment is walked 64 assignments
    // at a time; up to kPre chunks of expert ids are fetched ahead into
    // registers so one memory latency covers kPre chunks.
    constexpr int kPre = 16;
    for (int sb = a_begin; sb < a_end; sb += kPre * WAVE) {
        int ids[kPre];
#pragma unroll
        for (int q = 0; q < kPre; ++q) {
            const int a = sb + q * WAVE + lane;
            ids[q] = a < a_end ? eids[a] : 0;
        }
#pragma unroll
        for (int q = 0; q < kPre; ++q) {
            const int base = sb + q * WAVE;
            if (base >= a_end) break;
            const bool valid = base + lane < a_end;
            int rank, cnt;
            match_rank(ids[q], valid, nbits, &rank, &cnt);
            if (valid && rank == 0) my_hist[ids[q]] += cnt;
            __builtin_amdgcn_wave_barrier();
        }
    }
    __syncthreads();

    // per expert: prefix over segments, totals, scans, block map
    const int e = tid;
    int cnt = 0;
    if (e < E) {
        for (int w = 0; w < kGroupWaves; ++w) {
            const int h = s_hist[w * E + e];
            s_hist[w * E + e] = cnt;
            cnt += h;
        }
    }
    int total_rows, total_blocks;
    const int off = block_exclusive_scan(e < E ? cnt : 0, s_wave, &total_rows);
    const int nb = e < E ? (cnt + block_rows - 1) / block_rows : 0;
    const int bstart = block_exclusive_scan(nb, s_wave, &total_blocks);
    if (e < E) {
        r.counts[e] = cnt;
        r.offsets[e] = off;
        for (int i = 0; i < nb; ++i) {
            r.block_expert[bstart + i] = e;
            r.block_row[bstart + i] = off + block_rows * i;
        }
        for (int w = 0; w < kGroupWaves; ++w) s_hist[w * E + e] += off;
    }
    if (e == 0) {
        r.offsets[E] = total_rows;
        r.n_blocks[0] = total_blocks;
    }
    for (int b = total_blocks + tid; b < max_blocks; b += kGroupThreads) {
        r.block_expert[b] = -1;
        r.block_row[b] = -1;
    }
    __syncthreads();

    // pass 2: stable scatter (same walk; ranks continue from the segment bases)
    for (int sb = a_begin; sb < a_end; sb += kPre * WAVE) {
        int ids[kPre];
#pragma unroll
        for (int q = 0; q < kPre; ++q) {
            const int a = sb + q * WAVE + lane;
            ids[q] = a < a_end ? eids[a] : 0;
        }
#pragma unroll
        for (int q = 0; q < kPre; ++q) {
            const int base = sb + q * WAVE;
            if (base >= a_end) break;
            const int a = base + lane;
            const bool valid = a < a_end;
            const int ea = ids[q];
            int rank, c;
            match_rank(ea, valid, nbits, &rank, &c);
            int row = 0;
            if (valid) row = my_hist[ea] + rank;
            __builtin_amdgcn_wave_barrier();
            if (valid) {
                if (rank == 0) my_hist[ea] = row + c;
                r.sorted_assign[row] = a;
                r.assign_row[a] = row;
            }
            __builtin_amdgcn_wave_barrier();
        }
    }
}

__global__ __launch_bounds__(kGroupThreads) void route_group_kernel(
    const int32_t* __restrict__ topk_idx, int n, int E, int block_rows, int max_blocks,
    RoutingDev r) {
    extern __shared__ int smem_i[];
    group_all(topk_idx, n, E, block_rows, max_blocks, r, smem_i);
}

// Small T: every wave takes tokens wave, wave+16, ...; experts are kept in
// LDS for the grouping phase, so the whole routing is one launch.
template <int EPL>
__global__ __launch_bounds__(kGroupThreads) void route_fused_kernel(
    const float* __restrict__ logits, int T, int E, int k, int block_rows, int max_blocks,
    RoutingDev r) {
    extern __shared__ int smem_i[];
    const int wave = threadIdx.x / WAVE;
    int* s_hist = smem_i;                                  // kGroupWaves*E + kGroupWaves + 1
    int* s_eids = s_hist + kGroupWaves * E + kGroupWaves + 1;   // T*k
    uint32_t* s_scr = (uint32_t*)(s_eids + T * k) + wave * 3 * k;
    for (int t = wave; t < T; t += kGroupWaves) {
        topk_token<EPL>(logits + (size_t)t * E, E, k, r.topk_idx + (size_t)t * k,
                        r.topk_w + (size_t)t * k, s_scr, (int*)(s_scr + k),
                        (float*)(s_scr + 2 * k), s_eids + t * k);
    }
    __syncthreads();
    group_all(s_eids, T * k, E, block_rows, max_blocks, r, s_hist);
}

size_t route_ws_layout(int T, int E, int k, size_t* off_hist, size_t* off_rank) {
    (void)T;
    (void)E;
    (void)k;
    *off_hist = 0;
    *off_rank = 0;
    return 0;   // routing needs no device workspace beyond its outputs
}

static size_t group_lds_bytes(int E) {
    return (size_t)(kGroupWaves * E + kGroupWaves + 1) * sizeof(int);
}

static size_t fused_lds_bytes(int T, int E, int k) {
    return group_lds_bytes(E) + (size_t)T * k * sizeof(int) +
           (size_t)kGroupWaves * 3 * k * sizeof(uint32_t);
}

constexpr size_t kMaxLds = 64 * 1024;

hipError_t launch_route(const float* logits, int T, int E, int k, int block_rows, int max_blocks,
                        const RoutingDev& r, void* ws, hipStream_t stream) {
    (void)ws;
    const int epl = (E + WAVE - 1) / WAVE;
    const int n = T * k;
    if (T <= kFusedMaxTokens && fused_lds_bytes(T, E, k) <= kMaxLds) {
        const size_t smem = fused_lds_bytes(T, E, k);
#define MOE_FUSED(N)                                                                          \
    route_fused_kernel<N><<<1, kGroupThreads, smem, stream>>>(logits, T, E, k, block_rows,     \
                                                             max_blocks, r)
        if (epl <= 1) MOE_FUSED(1);
        else if (epl <= 2) MOE_FUSED(2);
        else if (epl <= 4) MOE_FUSED(4);
        else if (epl <= 8) MOE_FUSED(8);
        else MOE_FUSED(16);
#undef MOE_FUSED
        return hipGetLastError();
    }
    const size_t smem_t = (size_t)kTopkWaves * 3 * k * sizeof(uint32_t);
    const int grid = (T + kTopkWaves - 1) / kTopkWaves;
#define MOE_TOPK(N)                                                                         \
    route_topk_kernel<N><<<grid, kTopkWaves * WAVE, smem_t, stream>>>(logits, T, E, k,     \
                                                                      r.topk_idx, r.topk_w)
    if (epl <= 1) MOE_TOPK(1);
    else if (epl <= 2) MOE_TOPK(2);
    else if (epl <= 4) MOE_TOPK(4);
    else if (epl <= 8) MOE_TOPK(8);
    else MOE_TOPK(16);
#undef MOE_TOPK
    route_group_kernel<<<1, kGroupThreads, group_lds_bytes(E), stream>>>(
        r.topk_idx, n, E, block_rows, max_blocks, r);
    return hipGetLastError();
}

}  // namespace moeq4
