// Internal host-side interface between the C ABI (api.hip) and the kernel
// translation units.  Not part of the public ABI.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace moeq4 {

inline size_t align_up(size_t v, size_t a) { return (v + a - 1) / a * a; }

struct QMatDev {
    const uint32_t* codes;
    const uint16_t* scales;
    const uint16_t* biases;
    int layout;               // 0 = row-major code words, 1 = tile-packed (moe_q4_prepack),
                              // 2 = tile-packed with packed scale|bias words in `scales`
};

struct RoutingDev {
    int32_t* topk_idx;
    float* topk_w;
    int32_t* counts;
    int32_t* offsets;
    int32_t* sorted_assign;
    int32_t* assign_row;
    int32_t* block_expert;
    int32_t* block_row;
    int32_t* n_blocks;
};

// route.hip
int route_tokens_per_wg(int T, int k);
size_t route_ws_layout(int T, int E, int k, size_t* off_hist, size_t* off_rank);
hipError_t launch_route(const float* logits, int T, int E, int k, int block_rows, int max_blocks,
                        const RoutingDev& r, void* ws, hipStream_t stream);

// gemm_q4.hip
struct GemmProblem {
    const uint16_t* x;
    int T, H, I, I_sh, E, k, block_rows, max_blocks;
    RoutingDev r;
    QMatDev gate, up, down, sh_gate, sh_up, sh_down;
    uint16_t* expert_out;
    uint16_t* shared_out;
};
size_t gemm_ws_layout(int T, int I, int I_sh, int k, size_t* off_h, size_t* off_hsh);
hipError_t launch_gateup(const GemmProblem& p, void* ws, hipStream_t stream);
hipError_t launch_down(const GemmProblem& p, const void* ws, hipStream_t stream);
// weights expanded to bf16 [n_exp, N, K]: w = {gate, up, shared gate, shared up}
hipError_t launch_gateup_bf16(const GemmProblem& p, const uint16_t* const w[4], void* ws,
                              hipStream_t stream);
hipError_t launch_down_bf16(const GemmProblem& p, const uint16_t* down, const uint16_t* sh_down,
                            const void* ws, hipStream_t stream);

// dequant.hip
hipError_t launch_prepack(const uint32_t* src, int n_exp, int N, int K, uint32_t* dst,
                          hipStream_t stream);
hipError_t launch_pack_scales(const uint16_t* scales, const uint16_t* biases, int n_exp, int N,
                              int K, uint32_t* dst, hipStream_t stream);
hipError_t launch_dequant_bf16(const QMatDev& m, int n_exp, int N, int K, const int32_t* counts,
                               uint16_t* out, hipStream_t stream);

// decode.hip
struct DecodeArgs {
    const uint16_t* x;        // [1, H]
    const float* logits;      // [1, E]
    int H, I, I_sh, E, k;
    QMatDev gate, up, down, sh_gate, sh_up, sh_down;
    RoutingDev r;
    int write_routing;
    int max_blocks;
    uint16_t* h;              // workspace [k + 1][max(I, I_sh)] bf16: SwiGLU activations per slot
    int32_t* sel_idx;         // workspace [k]: chosen experts, slot order
    float* sel_w;             // workspace [k]: their weights
    uint16_t* y;              // [1, H]
};
// Workspace offsets (bytes) and size of one decode call.
struct DecodeWs {
    size_t h, sel_idx, sel_w, total;
};
DecodeWs decode_ws_layout(int H, int I, int I_sh, int k);
// (grid, threads) of the two decode launches.
void decode_launch_shapes(int H, int I, int I_sh, int k, int* grid1, int* threads1, int* grid2,
                          int* threads2);
hipError_t launch_decode(const DecodeArgs& args, hipStream_t stream);

// combine.hip
hipError_t launch_combine(const uint16_t* expert_out, const uint16_t* shared_out,
                          const float* shared_w, const int32_t* assign_row, const float* topk_w,
                          int T, int H, int k, uint16_t* y, hipStream_t stream);

// probe.hip: streaming-read probe, one sink word per 32 KB read
size_t read_probe_sink_words(size_t bytes);
hipError_t launch_read_probe(const void* buf, size_t bytes, uint32_t* sink, hipStream_t stream);
// probe.hip: chains of empty or dependent launches (kernel-boundary cost)
hipError_t launch_launch_probe(uint32_t* buf, int n_launches, int grid_a, int threads_a, int grid_b,
                               int threads_b, int dep, hipStream_t stream);

// router.hip
hipError_t launch_router(const uint16_t* x, int T, int H, const uint16_t* w_router, int E,
                         const uint16_t* w_gate, float* logits, float* gate, hipStream_t stream);

}  // namespace moeq4
