// Expansion of 4-bit groupwise-affine weights into a bf16 matrix in memory:
// the unfused layout that the pages measure the fused grouped GEMM against
// ([P2] aikraft.ru, "Technical optimizations: Prefill and Decode"; [P3]
// droneth.or.th, ablation paragraph: building the dequantization into the
// grouped GEMM instead was worth +77.4 % at 512 tokens).
//
// Each thread expands one code word (8 weights) with the same arithmetic as
// the fused GEMM (w = bf16_rne(fp32(q * s + b))) and stores 16 bytes; a
// workgroup covers 256 consecutive words, so loads and stores are coalesced.
// Experts whose routed count is zero are skipped when counts is given.
#include "moe_device.h"
#include "moe_launch.h"

namespace moeq4 {

constexpr int kDqThreads = 256;

__global__ __launch_bounds__(kDqThreads) void dequant_q4_bf16_kernel(
    QMatDev m, uint32_t words_per_exp, uint32_t words_per_row, uint32_t total_words,
    const int32_t* __restrict__ counts, uint16_t* __restrict__ out) {
    const uint32_t w = blockIdx.x * kDqThreads + threadIdx.x;
    if (w >= total_words) return;
    if (counts && counts[w / words_per_exp] == 0) return;
    const uint32_t row = w / words_per_row;            // expert * N + n
    const uint32_t grp = (w % words_per_row) / 8;      // 64-weight group of the word
    const uint32_t sidx = row * (words_per_row / 8) + grp;
    const float s = bf16_to_f32(m.scales[sidx]) * (1.0f / fp8_unit());
    const float b = bf16_to_f32(m.biases[sidx]);
    *(bf16x8_t*)(out + (size_t)w * 8) = dequant_word(m.codes[w], s, b);
}

hipError_t launch_dequant_bf16(const QMatDev& m, int n_exp, int N, int K, const int32_t* counts,
                               uint16_t* out, hipStream_t stream) {
    const uint32_t words_per_row = (uint32_t)(K / 8);
    const uint32_t words_per_exp = (uint32_t)N * words_per_row;
    const uint32_t total = (uint32_t)n_exp * words_per_exp;
    const uint32_t grid = (total + kDqThreads - 1) / kDqThreads;
    dequant_q4_bf16_kernel<<<grid, kDqThreads, 0, stream>>>(m, words_per_exp, words_per_row, total,
                                                           counts, out);
    return hipGetLastError();
}

}  // namespace moeq4
