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

// Lanes of a 64-lane chunk holding the same expert as this lane (expert ids
// below 2^kExpertBits; E <= 1000).  Bits at or above nbits are zero in every
// id, so the loop stops there.
constexpr int kExpertBits = 10;
__device__ __forceinline__ uint64_t match_mask(int e, bool valid, int nbits) {
    uint64_t match = __ballot(valid);
#pragma unroll
    for (int bit = 0; bit < kExpertBits; ++bit) {
        if (bit >= nbits) break;   // uniform
        const bool set = (e >> bit) & 1;
        const uint64_t bal = __ballot(valid && set);
        match &= set ? bal : ~bal;
    }
    return match;
}

// Inclusive sum over the wave's lanes.  DPP row_shr 1, 2, 4, 8 scan each
// 16-lane row; row_bcast 15 then adds row 0's total into row 1 (and row 2's
// into row 3), row_bcast 31 the first two rows' total into rows 2 and 3.
// Lanes without a source (or in rows the mask leaves out) add 0.
__device__ __forceinline__ int wave_incl_sum(int v) {
#define MOE_DPP_ADD(ctrl, rows) v += __builtin_amdgcn_update_dpp(0, v, ctrl, rows, 0xf, false)
    MOE_DPP_ADD(0x111, 0xf);   // row_shr:1
    MOE_DPP_ADD(0x112, 0xf);   // row_shr:2
    MOE_DPP_ADD(0x114, 0xf);   // row_shr:4
    MOE_DPP_ADD(0x118, 0xf);   // row_shr:8
    MOE_DPP_ADD(0x142, 0xa);   // row_bcast:15 into rows 1 and 3
    MOE_DPP_ADD(0x143, 0xc);   // row_bcast:31 into rows 2 and 3
#undef MOE_DPP_ADD
    return v;
}

// Exclusive scan of two values per thread over a kGroupThreads workgroup
// (s_wave: 2 * (kGroupWaves + 1) ints).  Returns the scans of a and b and
// both totals.
__device__ void block_exclusive_scan2(int a, int b, int* s_wave, int* ex_a, int* ex_b,
                                      int* tot_a, int* tot_b) {
    const int tid = threadIdx.x, lane = tid % WAVE, wave = tid / WAVE;
    const int ia = wave_incl_sum(a);
    const int ib = wave_incl_sum(b);
    if (lane == WAVE - 1) {
        s_wave[wave] = ia;
        s_wave[kGroupWaves + 1 + wave] = ib;
    }
    __syncthreads();
    if (wave == 0) {
        const int wa = lane < kGroupWaves ? s_wave[lane] : 0;
        const int wb = lane < kGroupWaves ? s_wave[kGroupWaves + 1 + lane] : 0;
        const int xa = wave_incl_sum(wa);
        const int xb = wave_incl_sum(wb);
        if (lane < kGroupWaves) {
            s_wave[lane] = xa - wa;
            s_wave[kGroupWaves + 1 + lane] = xb - wb;
        }
        if (lane == kGroupWaves - 1) {
            s_wave[kGroupWaves] = xa;
            s_wave[2 * kGroupWaves + 1] = xb;
        }
    }
    __syncthreads();
    *ex_a = s_wave[wave] + ia - a;
    *ex_b = s_wave[kGroupWaves + 1 + wave] + ib - b;
    *tot_a = s_wave[kGroupWaves];
    *tot_b = s_wave[2 * kGroupWaves + 1];
    __syncthreads();
}

// LDS of the grouping pass, in ints: the per-wave histograms and the scan's
// wave totals.
__host__ __device__ constexpr int group_lds_ints(int E) {
    return kGroupWaves * E + 2 * (kGroupWaves + 1);
}

// Blocks an expert's own thread writes into the block map; an expert with more
// (a hot expert of a skewed batch: 60-odd blocks) has them written by its whole
// wave, 64 at a time, instead of one thread's serial stores (3 us of a skewed
// chunk's grouping).
constexpr int kSerialBlocks = 8;

// Per expert: prefix of the kGroupWaves segment counts in s_hist, totals
// (counts), exclusive scan (offsets), the block map and n_blocks; afterwards
// s_hist[w * E + e] holds the first row of segment w's assignments to e.
__device__ void group_scan_block_map(int E, int block_rows, int max_blocks, const RoutingDev& r,
                                     int* s_hist) {
    const int tid = threadIdx.x, lane = tid % WAVE;
    int* s_wave = s_hist + kGroupWaves * E;
    const int e = tid;
    int h[kGroupWaves];
#pragma unroll
    for (int w = 0; w < kGroupWaves; ++w) h[w] = e < E ? s_hist[w * E + e] : 0;
    int cnt = 0;
#pragma unroll
    for (int w = 0; w < kGroupWaves; ++w) cnt += h[w];
    const int nb = e < E ? (cnt + block_rows - 1) / block_rows : 0;
    int off, bstart, total_rows, total_blocks;
    block_exclusive_scan2(cnt, nb, s_wave, &off, &bstart, &total_rows, &total_blocks);
    if (e < E) {
        r.counts[e] = cnt;
        r.offsets[e] = off;
        if (nb <= kSerialBlocks) {
            for (int i = 0; i < nb; ++i) {
                r.block_expert[bstart + i] = e;
                r.block_row[bstart + i] = off + block_rows * i;
            }
        }
        int run = off;
#pragma unroll
        for (int w = 0; w < kGroupWaves; ++w) {
            s_hist[w * E + e] = run;
            run += h[w];
        }
    }
    for (uint64_t hot = __ballot(e < E && nb > kSerialBlocks); hot; hot &= hot - 1) {
        const int src = __builtin_ctzll(hot);   // uniform: one hot expert of this wave
        const int he = __shfl(e, src, WAVE), hb = __shfl(bstart, src, WAVE);
        const int hn = __shfl(nb, src, WAVE), ho = __shfl(off, src, WAVE);
        for (int i = lane; i < hn; i += WAVE) {
            r.block_expert[hb + i] = he;
            r.block_row[hb + i] = ho + block_rows * i;
        }
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
}

// Histogram, scan, block map and stable scatter of n = T*k assignments
// whose experts are eids[0..n).  Needs kGroupThreads threads and
// kGroupWaves*E + 2*(kGroupWaves+1) ints of LDS at s_hist.
//
// Wave w owns the contiguous segment w of the assignments and walks it 64 at
// a time.  Inside a chunk, lanes with equal experts are found by ballots over
// the expert-id bits; the lowest such lane (the leader) speaks for them.
// Pass 1: leaders add their group's size to the wave's LDS histogram.  Pass 2:
// leaders take their group's first row with a returning LDS add on the
// running per-expert row (seeded with offset + the rows of lower segments)
// and hand it to their group; a lane's row is that plus its rank among equal
// experts in lower lanes.  A wave's LDS operations execute in program order,
// so rows follow assignment order within each expert: a stable counting
// sort.  When a segment fits in one batch of kPre chunks, its expert ids and
// match masks stay in registers between the two passes.
__device__ void group_all(const int32_t* eids, int n, int E, int block_rows, int max_blocks,
                          const RoutingDev& r, int* s_hist, int* s_sorted = nullptr) {
    constexpr int kPre = 16;
    const int tid = threadIdx.x, lane = tid % WAVE, wave = tid / WAVE;
    const int nbits = E > 1 ? 32 - __builtin_clz((unsigned)(E - 1)) : 0;
    const int seg = (n + kGroupWaves - 1) / kGroupWaves;
    const int a_begin = min(n, wave * seg), a_end = min(n, a_begin + seg);
    int* my_hist = s_hist + wave * E;
    const uint64_t lt = lanemask_lt();

    for (int i = tid; i < kGroupWaves * E; i += kGroupThreads) s_hist[i] = 0;
    __syncthreads();

    auto load_ids = [&](int sb, int (&ids)[kPre]) {
#pragma unroll
        for (int q = 0; q < kPre; ++q) {
            const int a = sb + q * WAVE + lane;
            ids[q] = a < a_end ? eids[a] : 0;
        }
    };
    auto count = [&](int sb, const int (&ids)[kPre], uint64_t (&mm)[kPre]) {
#pragma unroll
        for (int q = 0; q < kPre; ++q) {
            const int base = sb + q * WAVE;
            if (base >= a_end) break;
            const bool valid = base + lane < a_end;
            mm[q] = match_mask(ids[q], valid, nbits);
            if (valid && (mm[q] & lt) == 0) atomicAdd(&my_hist[ids[q]], __popcll(mm[q]));
        }
    };
    auto scatter = [&](int sb, const int (&ids)[kPre], const uint64_t (&mm)[kPre]) {
#pragma unroll
        for (int q = 0; q < kPre; ++q) {
            const int base = sb + q * WAVE;
            if (base >= a_end) break;
            const int a = base + lane;
            const bool valid = a < a_end;
            const uint64_t m = mm[q];
            int first = 0;
            if (valid && (m & lt) == 0) first = atomicAdd(&my_hist[ids[q]], __popcll(m));
            const int leader = valid ? __builtin_ctzll(m) : lane;
            first = __shfl(first, leader, WAVE);
            if (valid) {
                const int row = first + __popcll(m & lt);
                if (s_sorted) s_sorted[row] = a;   // uniform (see group_all_info)
                else r.sorted_assign[row] = a;
                r.assign_row[a] = row;
            }
        }
    };

    // pass 1: per-segment histograms
    const bool one_batch = a_end - a_begin <= kPre * WAVE;   // uniform per wave
    int ids[kPre];
    uint64_t mm[kPre];
    if (one_batch) {
        load_ids(a_begin, ids);
        count(a_begin, ids, mm);
    } else {
        for (int sb = a_begin; sb < a_end; sb += kPre * WAVE) {
            load_ids(sb, ids);
            count(sb, ids, mm);
        }
    }
    __syncthreads();

    group_scan_block_map(E, block_rows, max_blocks, r, s_hist);
    // pass 2: stable scatter
    if (one_batch) {
        scatter(a_begin, ids, mm);
    } else {
        for (int sb = a_begin; sb < a_end; sb += kPre * WAVE) {
            load_ids(sb, ids);
            #pragma unroll
            for (int q = 0; q < kPre; ++q) {
                const int base = sb + q * WAVE;
                mm[q] = base < a_end ? match_mask(ids[q], base + lane < a_end, nbits) : 0;
            }
            scatter(sb, ids, mm);
        }
    }
    if (s_sorted) {
        __syncthreads();
        for (int i = tid; i < n; i += kGroupThreads) r.sorted_assign[i] = s_sorted[i];
    }
}

__global__ __launch_bounds__(kGroupThreads) void route_group_kernel(
    const int32_t* __restrict__ topk_idx, int n, int E, int block_rows, int max_blocks,
    int stage_off, RoutingDev r) {
    extern __shared__ int smem_i[];
    group_all(topk_idx, n, E, block_rows, max_blocks, r, smem_i,
              stage_off ? smem_i + stage_off : nullptr);
}

// k = 4, 8 or 16 with T above the one-launch size: the top-k kernel takes
// 64 / k tokens per workgroup, i.e. one 64-assignment chunk, and records each
// assignment's match information inside that chunk (the lane of the first
// equal expert, the rank among equal experts in lower lanes, the group size),
// so the one-workgroup grouping pass needs no ballots.  The chunks are those
// of group_all_info below: chunk c = assignments [64c, 64c + 64).

__device__ __forceinline__ uint32_t chunk_info(uint64_t match) {
    const uint32_t leader = (uint32_t)__builtin_ctzll(match);
    const uint32_t rank = (uint32_t)__popcll(match & lanemask_lt());
    const uint32_t size = (uint32_t)__popcll(match);
    return leader | (rank << 8) | (size << 16);
}

template <int EPL, int KK>
__global__ __launch_bounds__((WAVE / KK) * WAVE) void route_topk_chunk_kernel(
    const float* __restrict__ logits, int T, int E, int32_t* __restrict__ topk_idx,
    float* __restrict__ topk_w, uint32_t* __restrict__ info) {
    constexpr int TOK = WAVE / KK;   // tokens per workgroup: one 64-assignment chunk
    __shared__ uint32_t s_scr[TOK][3 * KK];
    __shared__ int s_chunk[WAVE];
    const int wave = threadIdx.x / WAVE, lane = threadIdx.x % WAVE;
    const int t = blockIdx.x * TOK + wave;
    if (t < T)
        topk_token<EPL>(logits + (size_t)t * E, E, KK, topk_idx + (size_t)t * KK,
                        topk_w + (size_t)t * KK, s_scr[wave], (int*)(s_scr[wave] + KK),
                        (float*)(s_scr[wave] + 2 * KK), s_chunk + wave * KK);
    __syncthreads();
    if (wave == 0) {
        const int a = blockIdx.x * WAVE + lane;
        const bool valid = a < T * KK;
        const int e = valid ? s_chunk[lane] : 0;
        const int nbits = E > 1 ? 32 - __builtin_clz((unsigned)(E - 1)) : 0;
        const uint64_t m = match_mask(e, valid, nbits);
        if (valid) info[a] = chunk_info(m);
    }
}

// group_all with the chunk match information precomputed: wave w owns the
// contiguous chunks w*seg .. of the assignments.  Pass 1: chunk leaders add
// their group's size to the wave's histogram.  Pass 2: leaders take their
// group's first row with a returning LDS add on the running per-expert row and
// hand it to the group; a lane's row is that plus its rank.  The rows are the
// same stable counting sort as group_all's.  With s_sorted (n entries of LDS)
// the permutation is built there and written out in order afterwards: one
// workgroup issuing a 4-byte store per assignment to scattered rows is limited
// by its store requests (about 2 per cycle; 7.9 us for 16384 assignments).
__device__ void group_all_info(const int32_t* eids, const uint32_t* info, int n, int E,
                               int block_rows, int max_blocks, const RoutingDev& r, int* s_hist,
                               int* s_sorted) {
    constexpr int kPre = 16;
    const int tid = threadIdx.x, lane = tid % WAVE, wave = tid / WAVE;
    const int n_chunks = (n + WAVE - 1) / WAVE;
    const int seg = (n_chunks + kGroupWaves - 1) / kGroupWaves;
    const int c_begin = min(n_chunks, wave * seg), c_end = min(n_chunks, c_begin + seg);
    int* my_hist = s_hist + wave * E;

    auto load = [&](int cb, int (&ids)[kPre], uint32_t (&inf)[kPre]) {
#pragma unroll
        for (int q = 0; q < kPre; ++q) {
            const int a = (cb + q) * WAVE + lane;
            const bool ok = cb + q < c_end && a < n;
            ids[q] = ok ? eids[a] : 0;
            inf[q] = ok ? info[a] : 0u;
        }
    };
    auto count = [&](int cb, const int (&ids)[kPre], const uint32_t (&inf)[kPre]) {
#pragma unroll
        for (int q = 0; q < kPre; ++q) {
            if (cb + q >= c_end) break;
            const int a = (cb + q) * WAVE + lane;
            if (a < n && (int)(inf[q] & 0xFFu) == lane) atomicAdd(&my_hist[ids[q]], (int)(inf[q] >> 16));
        }
    };
    auto scatter = [&](int cb, const int (&ids)[kPre], const uint32_t (&inf)[kPre]) {
#pragma unroll
        for (int q = 0; q < kPre; ++q) {
            if (cb + q >= c_end) break;
            const int a = (cb + q) * WAVE + lane;
            const bool valid = a < n;
            const int leader = valid ? (int)(inf[q] & 0xFFu) : lane;
            int first = 0;
            if (valid && leader == lane) first = atomicAdd(&my_hist[ids[q]], (int)(inf[q] >> 16));
            first = __shfl(first, leader, WAVE);
            if (valid) {
                const int row = first + (int)((inf[q] >> 8) & 0xFFu);
                if (s_sorted) s_sorted[row] = a;   // uniform
                else r.sorted_assign[row] = a;
                r.assign_row[a] = row;
            }
        }
    };

    const bool one_batch = c_end - c_begin <= kPre;   // uniform per wave
    int ids[kPre];
    uint32_t inf[kPre];
    if (one_batch) load(c_begin, ids, inf);
    // Each wave clears only its own histogram, while its loads are in flight;
    // a wave's LDS operations execute in program order, so its adds below
    // follow the clear without a barrier.
    for (int i = lane; i < E; i += WAVE) my_hist[i] = 0;
    if (one_batch) {
        count(c_begin, ids, inf);
    } else {
        for (int cb = c_begin; cb < c_end; cb += kPre) {
            load(cb, ids, inf);
            count(cb, ids, inf);
        }
    }
    __syncthreads();
    group_scan_block_map(E, block_rows, max_blocks, r, s_hist);
    if (one_batch) {
        scatter(c_begin, ids, inf);
    } else {
        for (int cb = c_begin; cb < c_end; cb += kPre) {
            load(cb, ids, inf);
            scatter(cb, ids, inf);
        }
    }
    if (s_sorted) {
        __syncthreads();
        for (int i = tid; i < n; i += kGroupThreads) r.sorted_assign[i] = s_sorted[i];
    }
}

__global__ __launch_bounds__(kGroupThreads) void route_group_info_kernel(
    const int32_t* __restrict__ topk_idx, const uint32_t* __restrict__ info, int n, int E,
    int block_rows, int max_blocks, int stage_off, RoutingDev r) {
    extern __shared__ int smem_i[];
    group_all_info(topk_idx, info, n, E, block_rows, max_blocks, r, smem_i,
                   stage_off ? smem_i + stage_off : nullptr);
}

// Small T: every wave takes tokens wave, wave+16, ...; experts are kept in
// LDS for the grouping phase, so the whole routing is one launch.
template <int EPL>
__global__ __launch_bounds__(kGroupThreads) void route_fused_kernel(
    const float* __restrict__ logits, int T, int E, int k, int block_rows, int max_blocks,
    RoutingDev r) {
    extern __shared__ int smem_i[];
    const int wave = threadIdx.x / WAVE;
    int* s_hist = smem_i;                                  // kGroupWaves*E + 2*(kGroupWaves+1)
    int* s_eids = s_hist + group_lds_ints(E);   // T*k
    uint32_t* s_scr = (uint32_t*)(s_eids + T * k) + wave * 3 * k;
    for (int t = wave; t < T; t += kGroupWaves) {
        topk_token<EPL>(logits + (size_t)t * E, E, k, r.topk_idx + (size_t)t * k,
                        r.topk_w + (size_t)t * k, s_scr, (int*)(s_scr + k),
                        (float*)(s_scr + 2 * k), s_eids + t * k);
    }
    __syncthreads();
    group_all(s_eids, T * k, E, block_rows, max_blocks, r, s_hist);
}

static size_t group_lds_bytes(int E) {
    return (size_t)group_lds_ints(E) * sizeof(int);
}

// The grouping-info kernel builds the permutation in LDS up to this many
// assignments (64 KB; 2048 tokens at k = 8).
constexpr int kStageMaxAssign = 16384;

static size_t fused_lds_bytes(int T, int E, int k) {
    return group_lds_bytes(E) + (size_t)T * k * sizeof(int) +
           (size_t)kGroupWaves * 3 * k * sizeof(uint32_t);
}

constexpr size_t kMaxLds = 64 * 1024;

static bool use_fused(int T, int E, int k) {
    return T <= kFusedMaxTokens && fused_lds_bytes(T, E, k) <= kMaxLds;
}

// k = 4, 8 or 16 outside the one-launch path (64 / k tokens per top-k
// workgroup, at most 16 waves): the top-k kernel records per-chunk match
// information for the grouping pass (T * k words of workspace).
static bool use_chunk_info(int T, int E, int k) {
    return (k == 4 || k == 8 || k == 16) && !use_fused(T, E, k);
}

size_t route_ws_layout(int T, int E, int k, size_t* off_hist, size_t* off_rank) {
    *off_hist = 0;
    *off_rank = 0;
    if (!use_chunk_info(T, E, k)) return 0;   // no device workspace beyond the outputs
    return align_up((size_t)T * k * sizeof(uint32_t), 256);
}

hipError_t launch_route(const float* logits, int T, int E, int k, int block_rows, int max_blocks,
                        const RoutingDev& r, void* ws, hipStream_t stream) {
    (void)ws;
    const int epl = (E + WAVE - 1) / WAVE;
    const int n = T * k;
    if (use_fused(T, E, k)) {
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
    if (use_chunk_info(T, E, k)) {
        uint32_t* info = (uint32_t*)ws;
        const int tok = WAVE / k;
        const int grid_c = (T + tok - 1) / tok;
#define MOE_TOPK_CHUNK(N, KK)                                                                 \
    route_topk_chunk_kernel<N, KK><<<grid_c, tok * WAVE, 0, stream>>>(logits, T, E, r.topk_idx, \
                                                                       r.topk_w, info)
#define MOE_TOPK_CHUNK_K(KK)                          \
        if (epl <= 1) MOE_TOPK_CHUNK(1, KK);          \
        else if (epl <= 2) MOE_TOPK_CHUNK(2, KK);     \
        else if (epl <= 4) MOE_TOPK_CHUNK(4, KK);     \
        else if (epl <= 8) MOE_TOPK_CHUNK(8, KK);     \
        else MOE_TOPK_CHUNK(16, KK);
        if (k == 4) { MOE_TOPK_CHUNK_K(4) }
        else if (k == 8) { MOE_TOPK_CHUNK_K(8) }
        else { MOE_TOPK_CHUNK_K(16) }
#undef MOE_TOPK_CHUNK_K
#undef MOE_TOPK_CHUNK
        const bool stage = n <= kStageMaxAssign;
        const int stage_off = stage ? (int)(group_lds_bytes(E) / sizeof(int)) : 0;
        route_group_info_kernel<<<1, kGroupThreads,
                                  group_lds_bytes(E) + (stage ? (size_t)n * sizeof(int) : 0),
                                  stream>>>(r.topk_idx, info, n, E, block_rows, max_blocks,
                                            stage_off, r);
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
    const bool stage = n <= kStageMaxAssign;
    const int stage_off = stage ? (int)(group_lds_bytes(E) / sizeof(int)) : 0;
    route_group_kernel<<<1, kGroupThreads,
                         group_lds_bytes(E) + (stage ? (size_t)n * sizeof(int) : 0), stream>>>(
        r.topk_idx, n, E, block_rows, max_blocks, stage_off, r);
    return hipGetLastError();
}

}  // namespace moeq4
