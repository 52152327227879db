// Weighted combine of the routed expert outputs plus the shared expert:
// y[t] = sum_j topk_w[t, j] * expert_out[assign_row[t*k + j]] + g[t] * shared_out[t],
// fp32 sums in slot order with the shared expert last, one bf16 rounding.
// The shared expert processes every token ([P1] dothoosh.com Lily article,
// "Model specification"; [P3] droneth.or.th, "A big model ..."); the pages
// name no gate for it, so g = 1 unless an optional per-token gate is given
// (fma with g = 1 is exactly the plain sum).
#include "moe_device.h"
#include "moe_launch.h"

namespace moeq4 {

// One workgroup per token.  The token's k (row, weight) pairs are staged in
// LDS once; each thread then owns 8 consecutive columns per pass and issues
// its k 16-byte row gathers back to back before summing in slot order.
constexpr int kCombineThreads = 256;
constexpr int kCombineBatch = 8;   // gathers in flight per thread

__global__ __launch_bounds__(kCombineThreads) void combine_kernel(
    const uint16_t* __restrict__ expert_out, const uint16_t* __restrict__ shared_out,
    const int32_t* __restrict__ assign_row, const float* __restrict__ topk_w,
    const float* __restrict__ shared_w, int H, int k, uint16_t* __restrict__ y) {
    extern __shared__ int s_rw[];   // [k] rows, then [k] weights
    int* s_row = s_rw;
    float* s_w = (float*)(s_rw + k);
    const int t = blockIdx.x;
    for (int j = threadIdx.x; j < k; j += kCombineThreads) {
        s_row[j] = assign_row[(size_t)t * k + j];
        s_w[j] = topk_w[(size_t)t * k + j];
    }
    __syncthreads();
    for (int c = threadIdx.x * 8; c < H; c += kCombineThreads * 8) {
        float acc[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
        for (int j0 = 0; j0 < k; j0 += kCombineBatch) {
            u32x4_t v[kCombineBatch];
#pragma unroll
            for (int j = 0; j < kCombineBatch; ++j)
                if (j0 + j < k) v[j] = *(const u32x4_t*)(expert_out + (size_t)s_row[j0 + j] * H + c);
#pragma unroll
            for (int j = 0; j < kCombineBatch; ++j) {
                if (j0 + j >= k) break;
                const float w = s_w[j0 + j];
#pragma unroll
                for (int q = 0; q < 4; ++q) {
                    acc[2 * q] = __builtin_fmaf(w, __builtin_bit_cast(float, v[j][q] << 16), acc[2 * q]);
                    acc[2 * q + 1] =
                        __builtin_fmaf(w, __builtin_bit_cast(float, v[j][q] & 0xFFFF0000u), acc[2 * q + 1]);
                }
            }
        }
        if (shared_out) {
            const float g = shared_w ? shared_w[t] : 1.0f;
            const u32x4_t v = *(const u32x4_t*)(shared_out + (size_t)t * H + c);
#pragma unroll
            for (int q = 0; q < 4; ++q) {
                acc[2 * q] = __builtin_fmaf(g, __builtin_bit_cast(float, v[q] << 16), acc[2 * q]);
                acc[2 * q + 1] =
                    __builtin_fmaf(g, __builtin_bit_cast(float, v[q] & 0xFFFF0000u), acc[2 * q + 1]);
            }
        }
        u32x4_t o;
#pragma unroll
        for (int q = 0; q < 4; ++q) o[q] = pack_bf16x2(acc[2 * q], acc[2 * q + 1]);
        *(u32x4_t*)(y + (size_t)t * H + c) = o;
    }
}

hipError_t launch_combine(const uint16_t* expert_out, const uint16_t* shared_out,
                          const float* shared_w, const int32_t* assign_row, const float* topk_w,
                          int T, int H, int k, uint16_t* y, hipStream_t stream) {
    combine_kernel<<<T, kCombineThreads, (size_t)2 * k * sizeof(int), stream>>>(
        expert_out, shared_out, assign_row, topk_w, shared_w, H, k, y);
    return hipGetLastError();
}

}  // namespace moeq4
