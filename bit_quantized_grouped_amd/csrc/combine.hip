// Weighted combine of the routed expert outputs plus the shared expert:
// y[t] = sum_j topk_w[t, j] * expert_out[assign_row[t*k + j]] + shared_out[t],
// fp32 sums in slot order with the shared expert last, one bf16 rounding.
// The shared expert processes every token ([P1] dothoosh.com Lily article,
// "Model specification"; [P3] droneth.or.th, "A big model ..."); the pages
// name no gate for it, so it enters with weight 1.
#include "moe_device.h"
#include "moe_launch.h"

namespace moeq4 {

// One workgroup per token; each thread owns 8 consecutive columns per pass
// (16-byte loads of every routed row it gathers).
__global__ __launch_bounds__(256) void combine_kernel(
    const uint16_t* __restrict__ expert_out, const uint16_t* __restrict__ shared_out,
    const int32_t* __restrict__ assign_row, const float* __restrict__ topk_w, int H, int k,
    uint16_t* __restrict__ y) {
    const int t = blockIdx.x;
    for (int c = threadIdx.x * 8; c < H; c += 256 * 8) {
        float acc[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
        for (int j = 0; j < k; ++j) {
            const int row = assign_row[(size_t)t * k + j];
            const float w = topk_w[(size_t)t * k + j];
            const u32x4_t v = *(const u32x4_t*)(expert_out + (size_t)row * H + c);
#pragma unroll
            for (int q = 0; q < 4; ++q) {
                acc[2 * q] = __builtin_fmaf(w, __builtin_bit_cast(float, v[q] << 16), acc[2 * q]);
                acc[2 * q + 1] = __builtin_fmaf(w, __builtin_bit_cast(float, v[q] & 0xFFFF0000u), acc[2 * q + 1]);
            }
        }
        if (shared_out) {
            const u32x4_t v = *(const u32x4_t*)(shared_out + (size_t)t * H + c);
#pragma unroll
            for (int q = 0; q < 4; ++q) {
                acc[2 * q] += __builtin_bit_cast(float, v[q] << 16);
                acc[2 * q + 1] += __builtin_bit_cast(float, v[q] & 0xFFFF0000u);
            }
        }
        u32x4_t o;
#pragma unroll
        for (int q = 0; q < 4; ++q) o[q] = pack_bf16x2(acc[2 * q], acc[2 * q + 1]);
        *(u32x4_t*)(y + (size_t)t * H + c) = o;
    }
}

hipError_t launch_combine(const uint16_t* expert_out, const uint16_t* shared_out,
                          const int32_t* assign_row, const float* topk_w, int T, int H, int k,
                          uint16_t* y, hipStream_t stream) {
    combine_kernel<<<T, 256, 0, stream>>>(expert_out, shared_out, assign_row, topk_w, H, k, y);
    return hipGetLastError();
}

}  // namespace moeq4
