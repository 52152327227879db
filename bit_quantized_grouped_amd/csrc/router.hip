// Router projection: the scores the top-k selection runs on ([P1]
// dothoosh.com Lily article, "Model specification": a router scores the 256
// experts of every token and keeps 8).
//   logits[t, e] = sum_h x[t, h] * W_r[e, h]   (bf16 in, fp32 accumulation)
// and, when a gate row w_g is given, the per-token shared-expert weight
//   gate[t] = sigmoid(sum_h x[t, h] * w_g[h])
// computed as one more output row of the same product.
//
// A workgroup owns 16 tokens x 16 output rows; its 8 waves split the K range
// (32-wide steps, round robin) and sum their v_mfma_f32_16x16x32_bf16
// accumulators through LDS.  Both operands are read straight from memory in
// the MFMA layout: lane l supplies x[t0 + l%16][k0 + 8(l/16) .. +8] and
// W_r[r0 + l%16][same k], 16 bytes each.  Rows past T or past the last output
// row are clamped to a valid row and never stored.
#include "moe_device.h"
#include "moe_launch.h"

namespace moeq4 {

constexpr int kRtWaves = 8;
constexpr int kRtUnroll = 8;   // K steps whose loads a wave issues together

__global__ __launch_bounds__(kRtWaves * WAVE) void router_kernel(
    const uint16_t* __restrict__ x, int T, int H, const uint16_t* __restrict__ w_router, int E,
    const uint16_t* __restrict__ w_gate, float* __restrict__ logits, float* __restrict__ gate) {
    __shared__ f32x4_t s_acc[kRtWaves][WAVE];
    const int tid = threadIdx.x, lane = tid % WAVE;
    const int wave = __builtin_amdgcn_readfirstlane(tid / WAVE);
    const int nl = lane % 16, g = lane / 16;
    const int t0 = blockIdx.x * 16, r0 = blockIdx.y * 16;
    const int t = min(t0 + nl, T - 1);
    const int r = r0 + nl;
    const uint16_t* b_row = r < E ? w_router + (size_t)r * H
                          : (r == E && w_gate) ? w_gate
                                               : w_router + (size_t)(E - 1) * H;
    const uint16_t* a_row = x + (size_t)t * H;

    f32x4_t acc = {0.f, 0.f, 0.f, 0.f};
    const int steps = H / 32;
    for (int s0 = wave; s0 < steps; s0 += kRtWaves * kRtUnroll) {
        bf16x8_t a[kRtUnroll], b[kRtUnroll];
#pragma unroll
        for (int u = 0; u < kRtUnroll; ++u) {
            const int s = min(s0 + u * kRtWaves, steps - 1);   // clamped: re-read, not used
            a[u] = *(const bf16x8_t*)(a_row + s * 32 + 8 * g);
            b[u] = *(const bf16x8_t*)(b_row + s * 32 + 8 * g);
        }
#pragma unroll
        for (int u = 0; u < kRtUnroll; ++u)
            if (s0 + u * kRtWaves < steps) acc = mfma_16x16x32(a[u], b[u], acc);
    }
    s_acc[wave][lane] = acc;
    __syncthreads();
    if (wave != 0) return;
    f32x4_t sum = s_acc[0][lane];
#pragma unroll
    for (int w = 1; w < kRtWaves; ++w) {
        const f32x4_t o = s_acc[w][lane];
#pragma unroll
        for (int i = 0; i < 4; ++i) sum[i] += o[i];
    }
    // lane holds D[4g + i][nl]: token t0 + 4g + i, output row r
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        const int tt = t0 + 4 * g + i;
        if (tt >= T) continue;
        if (r < E) logits[(size_t)tt * E + r] = sum[i];
        else if (r == E && gate) gate[tt] = 1.0f / (1.0f + __expf(-sum[i]));
    }
}

hipError_t launch_router(const uint16_t* x, int T, int H, const uint16_t* w_router, int E,
                         const uint16_t* w_gate, float* logits, float* gate, hipStream_t stream) {
    const int rows = E + (w_gate ? 1 : 0);
    const dim3 grid((T + 15) / 16, (rows + 15) / 16);
    router_kernel<<<grid, kRtWaves * WAVE, 0, stream>>>(x, T, H, w_router, E, w_gate, logits,
                                                       gate);
    return hipGetLastError();
}

}  // namespace moeq4
