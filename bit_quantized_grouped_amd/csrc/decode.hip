// Batch-1 decode of the MoE layer in one launch per token.
//
// Decode is bound by bytes moved, not by compute ([P3] droneth.or.th,
// "Decode is limited by bandwidth more than by compute"), and the engine
// removes per-token host round trips and fuses kernel chains ([P1]
// dothoosh.com Lily article, "Decode optimizations", kernel-fusion bullet).
// One cooperative launch covers the whole layer for one token:
//   0. every workgroup selects the token's top-k from the logits itself
//      (the same deterministic selection as moe_route), so no barrier is
//      needed before the expert work; workgroup 0 writes the routing arrays;
//   1. gate/up rows of the k chosen experts and the shared expert are spread
//      over all waves: each wave streams whole weight rows (64 lanes x 16 B =
//      one 1 KB row of codes per load), dequantizes them in registers
//      (w = bf16_rne(fp32(q*s + b))), dots them with x in fp32 and
//      writes h = bf16(silu(g) * u);
//   -- one grid-wide barrier (all workgroups are co-resident) --
//   2. each wave owns output columns: for every expert it streams that
//      expert's down-projection row, dots it with h, and accumulates
//      topk_w * dot (shared expert with weight 1) in fp32; y = bf16(sum).
#include <hip/hip_cooperative_groups.h>

#include <atomic>

#include "moe_device.h"
#include "moe_launch.h"
#include "moe_topk.h"

namespace moeq4 {

namespace cg = cooperative_groups;

constexpr int kDecThreads = 512;
constexpr int kDecWaves = kDecThreads / WAVE;
constexpr int kDecMaxK = 64;

// Dot of 8 bf16 weights (packed pairs) with 8 bf16 activations (packed pairs):
// each bf16 is widened to fp32 exactly (its bits are the high half of the
// fp32) and the products are accumulated with fp32 FMAs.
__device__ __forceinline__ float dot8(const bf16x8_t& w, const u32x4_t& xv, float acc) {
    const u32x4_t wv = __builtin_bit_cast(u32x4_t, w);
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        acc = __builtin_fmaf(__builtin_bit_cast(float, wv[i] << 16),
                             __builtin_bit_cast(float, xv[i] << 16), acc);
        acc = __builtin_fmaf(__builtin_bit_cast(float, wv[i] & 0xFFFF0000u),
                             __builtin_bit_cast(float, xv[i] & 0xFFFF0000u), acc);
    }
    return acc;
}

__device__ __forceinline__ float wave_sum(float v) {
#pragma unroll
    for (int off = WAVE / 2; off >= 1; off >>= 1) v += shfl_xor(v, off);
    return v;
}

template <int EPL>
__global__ __launch_bounds__(kDecThreads) void decode_kernel(DecodeArgs p) {
    __shared__ int s_idx[kDecMaxK];
    __shared__ float s_w[kDecMaxK];
    __shared__ uint32_t s_scr[3 * kDecMaxK];
    const int tid = threadIdx.x, wave = tid / WAVE, lane = tid % WAVE;
    const int k = p.k, H = p.H;
    const float unit_inv = 1.0f / fp8_unit();

    // ---- 0. routing of the token (every workgroup, identical result) ----
    if (wave == 0)
        topk_token<EPL>(p.logits, p.E, k, s_idx, s_w, s_scr, (int*)(s_scr + k),
                        (float*)(s_scr + 2 * k), nullptr);
    __syncthreads();
    if (blockIdx.x == 0 && p.write_routing) {
        // T = 1: counts one-hot, rows in ascending expert order, one block per expert
        for (int e = tid; e < p.E; e += kDecThreads) p.r.counts[e] = 0;
        __syncthreads();
        if (tid < k) {
            const int e = s_idx[tid];
            int rank = 0;   // row of assignment tid = number of chosen experts below e
            for (int j = 0; j < k; ++j) rank += s_idx[j] < e ? 1 : 0;
            p.r.topk_idx[tid] = e;
            p.r.topk_w[tid] = s_w[tid];
            p.r.counts[e] = 1;
            p.r.sorted_assign[rank] = tid;
            p.r.assign_row[tid] = rank;
            p.r.block_expert[rank] = e;
            p.r.block_row[rank] = rank;
        }
        for (int e = tid; e <= p.E; e += kDecThreads) {
            int off = 0;
            for (int j = 0; j < k; ++j) off += s_idx[j] < e ? 1 : 0;
            p.r.offsets[e] = off;
        }
        for (int b = k + tid; b < p.max_blocks; b += kDecThreads) {
            p.r.block_expert[b] = -1;
            p.r.block_row[b] = -1;
        }
        if (tid == 0) p.r.n_blocks[0] = k;
    }

    const int gwave = blockIdx.x * kDecWaves + wave;
    const int nwaves = gridDim.x * kDecWaves;
    const int ldh = p.I > p.I_sh ? p.I : p.I_sh;

    // ---- 1. gate/up rows -> h ----
    const int n_routed = k * p.I;
    const int n_tasks = n_routed + p.I_sh;
    for (int task = gwave; task < n_tasks; task += nwaves) {
        const bool sh = task >= n_routed;
        const int j = sh ? k : task / p.I;
        const int n = sh ? task - n_routed : task % p.I;
        const int e = sh ? 0 : s_idx[j];
        const int N = sh ? p.I_sh : p.I;
        const QMatDev& g = sh ? p.sh_gate : p.gate;
        const QMatDev& u = sh ? p.sh_up : p.up;
        const size_t row = (size_t)e * N + n;
        float pg = 0.0f, pu = 0.0f;
        for (int kb = lane * 32; kb < H; kb += WAVE * 32) {
            const u32x4_t gw = *(const u32x4_t*)(g.codes + row * (H / 8) + kb / 8);
            const u32x4_t uw = *(const u32x4_t*)(u.codes + row * (H / 8) + kb / 8);
            const int grp = kb / 64;
            const float gs = bf16_to_f32(g.scales[row * (H / 64) + grp]) * unit_inv;
            const float gb = bf16_to_f32(g.biases[row * (H / 64) + grp]);
            const float us = bf16_to_f32(u.scales[row * (H / 64) + grp]) * unit_inv;
            const float ub = bf16_to_f32(u.biases[row * (H / 64) + grp]);
#pragma unroll
            for (int q = 0; q < 4; ++q) {
                const u32x4_t xv = *(const u32x4_t*)(p.x + kb + 8 * q);
                pg = dot8(dequant_word(gw[q], gs, gb), xv, pg);
                pu = dot8(dequant_word(uw[q], us, ub), xv, pu);
            }
        }
        pg = wave_sum(pg);
        pu = wave_sum(pu);
        if (lane == 0) p.h[(size_t)j * ldh + n] = __builtin_bit_cast(uint16_t, (__bf16)(silu_f32(pg) * pu));
    }

    cg::this_grid().sync();

    // ---- 2. down rows of every expert for this wave's columns, weighted sum ----
    const int half = lane / 32, lq = lane % 32;
    for (int cp = gwave; cp < H / 2; cp += nwaves) {
        const int c = 2 * cp + half;
        float acc = 0.0f;
        for (int j = 0; j <= k; ++j) {
            const bool sh = j == k;
            if (sh && !p.I_sh) break;
            const int N = sh ? p.I_sh : p.I;   // down K
            const int e = sh ? 0 : s_idx[j];
            const float wj = sh ? 1.0f : s_w[j];
            const QMatDev& d = sh ? p.sh_down : p.down;
            const size_t row = (size_t)e * H + c;
            float part = 0.0f;
            for (int wd = lq; wd < N / 8; wd += 32) {
                const uint32_t code = d.codes[row * (N / 8) + wd];
                const int grp = wd / 8;
                const float s = bf16_to_f32(d.scales[row * (N / 64) + grp]) * unit_inv;
                const float b = bf16_to_f32(d.biases[row * (N / 64) + grp]);
                const u32x4_t hv = *(const u32x4_t*)(p.h + (size_t)j * ldh + 8 * wd);
                part = dot8(dequant_word(code, s, b), hv, part);
            }
            acc = __builtin_fmaf(wj, part, acc);
        }
#pragma unroll
        for (int off = 16; off >= 1; off >>= 1) acc += shfl_xor(acc, off);
        if (lq == 0) p.y[c] = __builtin_bit_cast(uint16_t, (__bf16)acc);
    }
}

size_t decode_ws_bytes(int I, int I_sh, int k) {
    const int ldh = I > I_sh ? I : I_sh;
    return align_up((size_t)(k + 1) * ldh * sizeof(uint16_t), 256);
}

// Co-resident workgroups per CU for decode_kernel<EPL>, queried once per device.
template <int EPL>
static int decode_grid(int device) {
    // value depends only on the device and the kernel; benign if two threads compute it
    static std::atomic<int> cache[64];
    if (device < 0 || device >= 64) return 0;
    if (!cache[device].load(std::memory_order_relaxed)) {
        int per_cu = 0, cus = 0;
        if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&per_cu, decode_kernel<EPL>, kDecThreads, 0) !=
                hipSuccess ||
            hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, device) != hipSuccess)
            return 0;
        const int use = per_cu < 2 ? per_cu : 2;
        cache[device].store(use * cus, std::memory_order_relaxed);
    }
    return cache[device].load(std::memory_order_relaxed);
}

hipError_t launch_decode(const DecodeArgs& args, hipStream_t stream) {
    int device = 0;
    hipError_t e = hipGetDevice(&device);
    if (e != hipSuccess) return e;
    const int epl = (args.E + WAVE - 1) / WAVE;
    void* kargs[1] = {(void*)&args};
#define MOE_DECODE(N)                                                                         \
    do {                                                                                      \
        const int grid = decode_grid<N>(device);                                              \
        if (grid <= 0) return hipErrorInvalidConfiguration;                                   \
        return hipLaunchCooperativeKernel((const void*)decode_kernel<N>, dim3(grid),          \
                                          dim3(kDecThreads), kargs, 0, stream);               \
    } while (0)
    if (epl <= 1) MOE_DECODE(1);
    else if (epl <= 2) MOE_DECODE(2);
    else if (epl <= 4) MOE_DECODE(4);
    else if (epl <= 8) MOE_DECODE(8);
    else MOE_DECODE(16);
#undef MOE_DECODE
}

}  // namespace moeq4
