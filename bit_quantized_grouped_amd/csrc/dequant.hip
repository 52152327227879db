// Weight-format utilities: the load-time repack of code words into the
// tile-packed order and of scales and biases into packed scale|bias words,
// and the expansion of 4-bit groupwise-affine weights
// into a bf16 matrix in memory, the unfused layout that the pages measure
// the fused grouped GEMM against
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

// Code words into the tile-packed order (moe_q4_prepack, load time): each
// thread moves 4 consecutive words (16 bytes) of a row-major row to their
// place in the packed order, where they are again consecutive.
__global__ __launch_bounds__(kDqThreads) void prepack_kernel(const uint32_t* __restrict__ src,
                                                          uint32_t N, uint32_t K, uint32_t quads,
                                                          uint32_t* __restrict__ dst) {
    const uint32_t q = blockIdx.x * kDqThreads + threadIdx.x;
    if (q >= quads) return;
    const uint32_t w = q * 4;
    const uint32_t words_per_row = K / 8;
    const uint32_t row = w / words_per_row, c = w % words_per_row;   // row = e * N + n
    const uint32_t e = row / N, n = row % N;
    const size_t to = (size_t)e * N * words_per_row + code_word(1, n, c, K);
    *(u32x4_t*)(dst + to) = *(const u32x4_t*)(src + w);
}

// Scales and biases into the packed scale|bias order (moe_q4_pack_scales,
// load time): thread i writes word i of the packed array, i = ((n/64)*G +
// g)*64 + n%64 for global row n and group g, so the stores are coalesced.
__global__ __launch_bounds__(kDqThreads) void pack_scales_kernel(
    const uint16_t* __restrict__ scales, const uint16_t* __restrict__ biases, uint32_t G,
    uint32_t total, uint32_t* __restrict__ dst) {
    const uint32_t i = blockIdx.x * kDqThreads + threadIdx.x;
    if (i >= total) return;
    const uint32_t r = i % 64, g = (i / 64) % G, tile = i / (64 * G);
    const uint32_t src = (tile * 64 + r) * G + g;
    dst[i] = (uint32_t)scales[src] | ((uint32_t)biases[src] << 16);
}

hipError_t launch_pack_scales(const uint16_t* scales, const uint16_t* biases, int n_exp, int N,
                              int K, uint32_t* dst, hipStream_t stream) {
    const uint32_t total = (uint32_t)((size_t)n_exp * N * (K / 64));
    pack_scales_kernel<<<(total + kDqThreads - 1) / kDqThreads, kDqThreads, 0, stream>>>(
        scales, biases, (uint32_t)(K / 64), total, dst);
    return hipGetLastError();
}

hipError_t launch_prepack(const uint32_t* src, int n_exp, int N, int K, uint32_t* dst,
                          hipStream_t stream) {
    const uint32_t quads = (uint32_t)((size_t)n_exp * N * (K / 8) / 4);
    prepack_kernel<<<(quads + kDqThreads - 1) / kDqThreads, kDqThreads, 0, stream>>>(
        src, (uint32_t)N, (uint32_t)K, quads, dst);
    return hipGetLastError();
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
