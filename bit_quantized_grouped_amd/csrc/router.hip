// Router projection: the scores the top-k selection runs on ([P1]
// dothoosh.com Lily article, "Model specification": a router scores the 256
// experts of every token and keeps 8).
//   logits[t, e] = sum_h x[t, h] * W_r[e, h]   (bf16 in, fp32 accumulation)
// and, when a gate row w_g is given, the per-token shared-expert weight
//   gate[t] = sigmoid(sum_h x[t, h] * w_g[h])
// computed as one more output row of the same product.
//
// A workgroup owns TM tokens x TN output rows (16 x 16 below 384 tokens,
// 32 x 32 from there: the larger tile halves the L2 reads of x and W_r per
// output, the smaller keeps enough workgroups busy for short calls; at
// H = 2048 and 256 experts + gate, 16 x 16 is faster up to 256 tokens and
// 32 x 32 from 512).
// Its 8 waves split the K range (32-wide steps, round robin), each wave
// accumulating every 16 x 16 subtile with v_mfma_f32_16x16x32_bf16, and the
// wave partials are summed through LDS in a fixed order.  Both operands are
// read straight from memory in the MFMA layout: lane l supplies
// x[token + l%16][k0 + 8(l/16) .. +8] and W_r[row + l%16][same k], 16 bytes
// each.  Tokens past T or rows past the last output row are clamped to a
// valid row and never stored.
#include "moe_device.h"
#include "moe_launch.h"

namespace moeq4 {

template <int kTM, int kTN, int kRtWaves, int kRtUnroll>
__global__ __launch_bounds__(kRtWaves * WAVE) void router_kernel(
    const uint16_t* __restrict__ x, int T, int H, const uint16_t* __restrict__ w_router, int E,
    const uint16_t* __restrict__ w_gate, float* __restrict__ logits, float* __restrict__ gate) {
    constexpr int kMT = kTM / 16, kNT = kTN / 16;
    __shared__ f32x4_t s_acc[kRtWaves][kMT * kNT][WAVE];
    const int tid = threadIdx.x, lane = tid % WAVE;
    const int wave = __builtin_amdgcn_readfirstlane(tid / WAVE);
    const int nl = lane % 16, g = lane / 16;
    const int t0 = blockIdx.x * kTM, r0 = blockIdx.y * kTN;
    const uint16_t* a_row[kMT];
    const uint16_t* b_row[kNT];
#pragma unroll
    for (int mi = 0; mi < kMT; ++mi) a_row[mi] = x + (size_t)min(t0 + mi * 16 + nl, T - 1) * H;
#pragma unroll
    for (int ni = 0; ni < kNT; ++ni) {
        const int r = r0 + ni * 16 + nl;
        b_row[ni] = r < E ? w_router + (size_t)r * H
                  : (r == E && w_gate) ? w_gate
                                       : w_router + (size_t)(E - 1) * H;
    }
    f32x4_t acc[kMT][kNT];
#pragma unroll
    for (int mi = 0; mi < kMT; ++mi)
#pragma unroll
        for (int ni = 0; ni < kNT; ++ni) acc[mi][ni] = f32x4_t{0.f, 0.f, 0.f, 0.f};
    const int steps = H / 32;
    for (int s0 = wave; s0 < steps; s0 += kRtWaves * kRtUnroll) {
        bf16x8_t a[kRtUnroll][kMT], b[kRtUnroll][kNT];
#pragma unroll
        for (int u = 0; u < kRtUnroll; ++u) {
            const int s = min(s0 + u * kRtWaves, steps - 1);
#pragma unroll
            for (int mi = 0; mi < kMT; ++mi) a[u][mi] = *(const bf16x8_t*)(a_row[mi] + s * 32 + 8 * g);
#pragma unroll
            for (int ni = 0; ni < kNT; ++ni) b[u][ni] = *(const bf16x8_t*)(b_row[ni] + s * 32 + 8 * g);
        }
#pragma unroll
        for (int u = 0; u < kRtUnroll; ++u)
            if (s0 + u * kRtWaves < steps)
#pragma unroll
                for (int mi = 0; mi < kMT; ++mi)
#pragma unroll
                    for (int ni = 0; ni < kNT; ++ni)
                        acc[mi][ni] = mfma_16x16x32(a[u][mi], b[u][ni], acc[mi][ni]);
    }
#pragma unroll
    for (int mi = 0; mi < kMT; ++mi)
#pragma unroll
        for (int ni = 0; ni < kNT; ++ni) s_acc[wave][mi * kNT + ni][lane] = acc[mi][ni];
    __syncthreads();
    // wave w sums tiles w, w + kRtWaves, ... over the waves in a fixed order
    for (int tI = wave; tI < kMT * kNT; tI += kRtWaves) {
        f32x4_t sum = s_acc[0][tI][lane];
#pragma unroll
        for (int w = 1; w < kRtWaves; ++w) {
            const f32x4_t o = s_acc[w][tI][lane];
#pragma unroll
            for (int i = 0; i < 4; ++i) sum[i] += o[i];
        }
        const int mi = tI / kNT, ni = tI % kNT;
        const int r = r0 + ni * 16 + nl;
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const int tt = t0 + mi * 16 + 4 * g + i;
            if (tt >= T) continue;
            if (r < E) logits[(size_t)tt * E + r] = sum[i];
            else if (r == E && gate) gate[tt] = 1.0f / (1.0f + __expf(-sum[i]));
        }
    }
}

template <int TM, int TN, int WAVES, int UNROLL>
static void launch_router_tiles(const uint16_t* x, int T, int H, const uint16_t* w_router, int E,
                                const uint16_t* w_gate, float* logits, float* gate,
                                hipStream_t stream) {
    const int rows = E + (w_gate ? 1 : 0);
    const dim3 grid((T + TM - 1) / TM, (rows + TN - 1) / TN);
    router_kernel<TM, TN, WAVES, UNROLL><<<grid, WAVES * WAVE, 0, stream>>>(
        x, T, H, w_router, E, w_gate, logits, gate);
}

hipError_t launch_router(const uint16_t* x, int T, int H, const uint16_t* w_router, int E,
                         const uint16_t* w_gate, float* logits, float* gate, hipStream_t stream) {
    if (T >= 384)
        launch_router_tiles<32, 32, 8, 4>(x, T, H, w_router, E, w_gate, logits, gate, stream);
    else
        launch_router_tiles<16, 16, 8, 8>(x, T, H, w_router, E, w_gate, logits, gate, stream);
    return hipGetLastError();
}

}  // namespace moeq4
