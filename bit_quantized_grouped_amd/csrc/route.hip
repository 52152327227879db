// GPU-resident routing: top-k + softmax weights, expert histogram, exclusive
// prefix scan, stable scatter and the row-block map, with no host round trip
// ([P1] dothoosh.com Lily article, "Prefill optimizations", GPU-resident
// routing bullet; [P1] "Model specification": 256 experts, 8 selected).
//
// Three kernels on one stream:
//   route_topk   one wave per token: k rounds of wave arg-max over the
//                logits (ties to the lower expert), softmax over the k
//                chosen; then, per workgroup, a histogram of its
//                assignments and each assignment's rank among the
//                workgroup's earlier assignments to the same expert
//                (ballot match, scanned 64 assignments at a time, so the
//                rank order is ascending assignment index: a stable sort).
//   route_scan   one workgroup: per expert, the exclusive prefix over
//                workgroups (-> each workgroup's first row for that
//                expert), the totals (counts), their exclusive scan
//                (offsets), and the block map with the device-side n_blocks.
//   route_scatter  row = base[wg][e] + rank: sorted_assign and assign_row.
// Every output is a deterministic function of the logits.
#include "moe_device.h"
#include "moe_launch.h"

namespace moeq4 {

constexpr int kRouteThreads = 256;
constexpr int kRouteWaves = kRouteThreads / WAVE;

template <int EPL>
__global__ __launch_bounds__(kRouteThreads) void route_topk_kernel(
    const float* __restrict__ logits, int T, int E, int k, int tok_per_wg,
    int32_t* __restrict__ topk_idx, float* __restrict__ topk_w,
    int32_t* __restrict__ wg_hist, int32_t* __restrict__ local_rank) {
    extern __shared__ int32_t smem[];
    int32_t* s_exp = smem;                         // [tok_per_wg * k]
    float* s_val = (float*)(smem + tok_per_wg * k);   // [tok_per_wg * k]
    int32_t* s_cursor = smem + 2 * tok_per_wg * k;    // [E]

    const int tid = threadIdx.x;
    const int wave = tid / WAVE;
    const int lane = tid % WAVE;
    const int t0 = blockIdx.x * tok_per_wg;
    const int ntok = min(tok_per_wg, T - t0);

    for (int e = tid; e < E; e += kRouteThreads) s_cursor[e] = 0;

    for (int i = wave; i < ntok; i += kRouteWaves) {
        const int t = t0 + i;
        const float* row = logits + (size_t)t * E;
        float v[EPL];
#pragma unroll
        for (int j = 0; j < EPL; ++j) {
            const int e = lane + WAVE * j;
            v[j] = e < E ? row[e] + 0.0f : 0.0f;   // + 0.0f: -0.0 -> +0.0
        }
        uint32_t taken = 0;
        for (int r = 0; r < k; ++r) {
            float bv = 0.0f;
            int be = 0x7fffffff;
#pragma unroll
            for (int j = 0; j < EPL; ++j) {
                const int e = lane + WAVE * j;
                const bool ok = e < E && !((taken >> j) & 1u);
                if (ok && (be == 0x7fffffff || v[j] > bv)) {   // ascending e per lane: strict > keeps the lower index
                    bv = v[j];
                    be = e;
                }
            }
#pragma unroll
            for (int off = WAVE / 2; off >= 1; off >>= 1) {
                const float ov = shfl_xor(bv, off);
                const int oe = shfl_xor(be, off);
                const bool o_better = oe != 0x7fffffff &&
                                      (be == 0x7fffffff || ov > bv || (ov == bv && oe < be));
                if (o_better) {
                    bv = ov;
                    be = oe;
                }
            }
            if ((be % WAVE) == lane) taken |= 1u << (be / WAVE);
            if (lane == 0) {
                s_exp[i * k + r] = be;
                s_val[i * k + r] = bv;
            }
        }
    }
    __syncthreads();

    // softmax over the k chosen logits of each token (max = first chosen)
    for (int i = wave; i < ntok; i += kRouteWaves) {
        const float m = s_val[i * k];
        float part = 0.0f;
        for (int r = lane; r < k; r += WAVE) part += __expf(s_val[i * k + r] - m);
#pragma unroll
        for (int off = WAVE / 2; off >= 1; off >>= 1) part += shfl_xor(part, off);
        const float inv = 1.0f / part;
        const int t = t0 + i;
        for (int r = lane; r < k; r += WAVE) {
            topk_idx[(size_t)t * k + r] = s_exp[i * k + r];
            topk_w[(size_t)t * k + r] = __expf(s_val[i * k + r] - m) * inv;
        }
    }

    // Stable local ranks and the workgroup histogram: wave 0 walks the
    // workgroup's assignments in ascending order, 64 at a time.
    if (wave == 0) {
        const int n_asg = ntok * k;
        const int nbits = E > 1 ? 32 - __builtin_clz((unsigned)(E - 1)) : 0;
        const uint64_t lt = lanemask_lt();
        for (int base = 0; base < n_asg; base += WAVE) {
            const int a = base + lane;
            const bool valid = a < n_asg;
            const int e = valid ? s_exp[a] : 0;
            uint64_t match = __ballot(valid);
            for (int bit = 0; bit < nbits; ++bit) {
                const bool set = (e >> bit) & 1;
                const uint64_t bal = __ballot(valid && set);
                match &= set ? bal : ~bal;
            }
            const int rank = __popcll(match & lt);
            const int cnt = __popcll(match);
            int prev = 0;
            if (valid) prev = s_cursor[e];
            __builtin_amdgcn_wave_barrier();
            if (valid) {
                local_rank[(size_t)t0 * k + a] = prev + rank;
                if (rank == 0) s_cursor[e] = prev + cnt;
            }
            __builtin_amdgcn_wave_barrier();
        }
    }
    __syncthreads();
    for (int e = tid; e < E; e += kRouteThreads) wg_hist[(size_t)blockIdx.x * E + e] = s_cursor[e];
}

constexpr int kScanThreads = 1024;

// Exclusive scan of one value per thread over the workgroup (E <= 1024).
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
        const int nw = kScanThreads / WAVE;
        int w = lane < nw ? s_wave[lane] : 0;
        int wi = w;
#pragma unroll
        for (int off = 1; off < WAVE; off <<= 1) {
            const int o = __shfl_up(wi, off, WAVE);
            if (lane >= off) wi += o;
        }
        if (lane < nw) s_wave[lane] = wi - w;   // exclusive wave prefix
        if (lane == nw - 1) s_wave[nw] = wi;    // grand total
    }
    __syncthreads();
    const int res = s_wave[wave] + incl - v;
    *total = s_wave[kScanThreads / WAVE];
    __syncthreads();
    return res;
}

__global__ __launch_bounds__(kScanThreads) void route_scan_kernel(
    int32_t* __restrict__ wg_hist, int nwg, int E, int block_rows, int max_blocks,
    int32_t* __restrict__ counts, int32_t* __restrict__ offsets,
    int32_t* __restrict__ block_expert, int32_t* __restrict__ block_row,
    int32_t* __restrict__ n_blocks) {
    __shared__ int s_wave[kScanThreads / WAVE + 1];
    const int e = threadIdx.x;
    int cnt = 0;
    if (e < E) {
        // exclusive prefix over workgroups, in place
        for (int w = 0; w < nwg; ++w) {
            const int h = wg_hist[(size_t)w * E + e];
            wg_hist[(size_t)w * E + e] = cnt;
            cnt += h;
        }
    }
    int total_rows;
    const int off = block_exclusive_scan(e < E ? cnt : 0, s_wave, &total_rows);
    const int nb = e < E ? (cnt + block_rows - 1) / block_rows : 0;
    int total_blocks;
    const int bstart = block_exclusive_scan(nb, s_wave, &total_blocks);
    if (e < E) {
        counts[e] = cnt;
        offsets[e] = off;
        for (int i = 0; i < nb; ++i) {
            block_expert[bstart + i] = e;
            block_row[bstart + i] = off + block_rows * i;
        }
        for (int w = 0; w < nwg; ++w) wg_hist[(size_t)w * E + e] += off;
    }
    if (e == 0) {
        offsets[E] = total_rows;
        n_blocks[0] = total_blocks;
    }
    for (int b = total_blocks + e; b < max_blocks; b += kScanThreads) {
        block_expert[b] = -1;
        block_row[b] = -1;
    }
}

__global__ __launch_bounds__(256) void route_scatter_kernel(
    const int32_t* __restrict__ topk_idx, const int32_t* __restrict__ wg_base,
    const int32_t* __restrict__ local_rank, int n_asg, int E, int asg_per_wg,
    int32_t* __restrict__ sorted_assign, int32_t* __restrict__ assign_row) {
    const int a = blockIdx.x * 256 + threadIdx.x;
    if (a >= n_asg) return;
    const int e = topk_idx[a];
    const int w = a / asg_per_wg;
    const int row = wg_base[(size_t)w * E + e] + local_rank[a];
    sorted_assign[row] = a;
    assign_row[a] = row;
}

int route_tokens_per_wg(int T, int k) {
    // keep the per-workgroup assignment list and ranking walk short
    int tpw = 16;
    while (tpw > 1 && tpw * k > 4096) tpw >>= 1;
    (void)T;
    return tpw;
}

size_t route_ws_layout(int T, int E, int k, size_t* off_hist, size_t* off_rank) {
    const int tpw = route_tokens_per_wg(T, k);
    const size_t nwg = (size_t)(T + tpw - 1) / tpw;
    size_t o = 0;
    *off_hist = o;
    o += align_up(nwg * E * sizeof(int32_t), 256);
    *off_rank = o;
    o += align_up((size_t)T * k * sizeof(int32_t), 256);
    return o;
}

hipError_t launch_route(const float* logits, int T, int E, int k, int block_rows, int max_blocks,
                        const RoutingDev& r, void* ws, hipStream_t stream) {
    size_t off_hist, off_rank;
    route_ws_layout(T, E, k, &off_hist, &off_rank);
    int32_t* wg_hist = (int32_t*)((char*)ws + off_hist);
    int32_t* local_rank = (int32_t*)((char*)ws + off_rank);
    const int tpw = route_tokens_per_wg(T, k);
    const int nwg = (T + tpw - 1) / tpw;
    const size_t smem = (size_t)(2 * tpw * k + E) * sizeof(int32_t);
    const int epl = (E + WAVE - 1) / WAVE;
#define MOE_ROUTE_TOPK(N)                                                                     \
    route_topk_kernel<N><<<nwg, kRouteThreads, smem, stream>>>(logits, T, E, k, tpw,        \
                                                              r.topk_idx, r.topk_w, wg_hist, \
                                                              local_rank)
    if (epl <= 1) MOE_ROUTE_TOPK(1);
    else if (epl <= 2) MOE_ROUTE_TOPK(2);
    else if (epl <= 4) MOE_ROUTE_TOPK(4);
    else if (epl <= 8) MOE_ROUTE_TOPK(8);
    else MOE_ROUTE_TOPK(16);
#undef MOE_ROUTE_TOPK
    route_scan_kernel<<<1, kScanThreads, 0, stream>>>(wg_hist, nwg, E, block_rows, max_blocks,
                                                      r.counts, r.offsets, r.block_expert,
                                                      r.block_row, r.n_blocks);
    const int n_asg = T * k;
    route_scatter_kernel<<<(n_asg + 255) / 256, 256, 0, stream>>>(
        r.topk_idx, wg_hist, local_rank, n_asg, E, tpw * k, r.sorted_assign, r.assign_row);
    return hipGetLastError();
}

}  // namespace moeq4
