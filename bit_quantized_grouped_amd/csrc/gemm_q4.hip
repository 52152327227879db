// Grouped expert GEMM with the 4-bit dequantization fused into the tiles
// ([P1] dothoosh.com Lily article, "Prefill optimizations", fused
// dequantization bullet; [P3] droneth.or.th, "A big model that touches only
// part of its weights per token": weights are rebuilt tile by tile inside the
// grouped GEMM as bf16 and accumulated in FP32; expanded weights never reach
// memory).
//
// One kernel template serves both projections:
//   NMAT = 2  gate and up over the same 16 output columns per wave, SwiGLU
//             epilogue h = silu(g) * u -> bf16 h  (A = x rows gathered by token)
//   NMAT = 1  down projection -> bf16 expert_out / shared_out
//             (A = h rows, contiguous in sorted-row order)
// Work unit = one row block of the block map (MT rows of one expert) x 64
// output columns (4 waves x 16).  The shared expert is an extra dense group
// over all tokens, as the first sh_blocks slots of grid.y.
//
// Data path per K-chunk of KC:
//   A: the block's MT rows x KC bf16 are staged in LDS (row stride KC+8 to
//      keep ds_read_b128 conflict free) and read once per MFMA by every wave;
//   B: each lane loads KC/32 consecutive code words of one weight row
//      straight from HBM into registers (4 lanes cover a row's KC/2 bytes
//      contiguously), dequantizes one word (8 weights) at a time to bf16 in
//      registers and feeds it to v_mfma_f32_16x16x32_bf16.  A lane's 8
//      weights are the 8 consecutive k of one code word, so the K order
//      inside each MFMA is the natural one for both operands.
#include "moe_device.h"
#include "moe_launch.h"

namespace moeq4 {

struct GroupedArgs {
    const uint16_t* a_routed;
    const uint16_t* a_shared;
    int lda_routed, lda_shared;
    int gather;            // routed A rows: 1 -> token sorted_assign[row]/k, 0 -> row itself
    int k;
    int T;
    const int32_t* sorted_assign;
    const int32_t* block_expert;
    const int32_t* block_row;
    const int32_t* n_blocks;
    const int32_t* offsets;
    int sh_blocks;
    QMatDev rB[2];
    QMatDev sB[2];
    int N, K, N_sh, K_sh;
    uint16_t* out_routed;
    uint16_t* out_shared;
};

template <int NMAT, int MT, int KC>
__global__ __launch_bounds__(256) void grouped_q4_kernel(GroupedArgs p) {
    constexpr int W = KC / 32;       // code words per lane per chunk
    constexpr int MSUB = MT / 16;
    constexpr int LDA = KC + 8;
    __shared__ __attribute__((aligned(16))) uint16_t sA[MT * LDA];
    __shared__ int s_row[MT];

    const int tid = threadIdx.x;
    const int wave = tid >> 6, lane = tid & 63;
    const int nl = lane & 15, g = lane >> 4;
    const int slot = blockIdx.y;
    const bool is_sh = slot < p.sh_blocks;

    int r0, nr, N, K, lda, expert = 0;
    const uint16_t* A;
    uint16_t* out;
    if (is_sh) {
        r0 = slot * MT;
        nr = min(MT, p.T - r0);
        N = p.N_sh;
        K = p.K_sh;
        A = p.a_shared;
        lda = p.lda_shared;
        out = p.out_shared;
    } else {
        const int b = slot - p.sh_blocks;
        if (b >= p.n_blocks[0]) return;
        expert = p.block_expert[b];
        r0 = p.block_row[b];
        nr = min(MT, p.offsets[expert + 1] - r0);
        N = p.N;
        K = p.K;
        A = p.a_routed;
        lda = p.lda_routed;
        out = p.out_routed;
    }
    if ((int)blockIdx.x * 64 >= N) return;   // uniform per workgroup

    if (tid < MT) {
        const int rr = min(tid, nr - 1);   // padding rows repeat the last row; never stored
        s_row[tid] = (is_sh || !p.gather) ? r0 + rr : p.sorted_assign[r0 + rr] / p.k;
    }

    const int n = blockIdx.x * 64 + wave * 16 + nl;   // this lane's weight row
    const uint32_t* bc[NMAT];
    const uint16_t* bs[NMAT];
    const uint16_t* bb[NMAT];
#pragma unroll
    for (int m = 0; m < NMAT; ++m) {
        const QMatDev& q = is_sh ? p.sB[m] : p.rB[m];
        const size_t row = (size_t)expert * N + n;
        bc[m] = q.codes + row * (K / 8) + g * W;
        bs[m] = q.scales + row * (K / 64);
        bb[m] = q.biases + row * (K / 64);
    }
    const float unit_inv = 1.0f / fp8_unit();

    f32x4_t acc[NMAT][MSUB];
#pragma unroll
    for (int m = 0; m < NMAT; ++m)
#pragma unroll
        for (int i = 0; i < MSUB; ++i) acc[m][i] = f32x4_t{0.f, 0.f, 0.f, 0.f};

    __syncthreads();
    const int nchunks = K / KC;
    for (int c = 0; c < nchunks; ++c) {
        uint32_t wv[NMAT][W];
        float s[NMAT], bz[NMAT];
        const int grp = (c * KC + g * (KC / 4)) / 64;
#pragma unroll
        for (int m = 0; m < NMAT; ++m) {
            const uint32_t* src = bc[m] + c * (KC / 8);
            if constexpr (W >= 4) {
#pragma unroll
                for (int j = 0; j < W; j += 4) {
                    const u32x4_t v = *(const u32x4_t*)(src + j);
                    wv[m][j] = v[0];
                    wv[m][j + 1] = v[1];
                    wv[m][j + 2] = v[2];
                    wv[m][j + 3] = v[3];
                }
            } else {
                const u32x2_t v = *(const u32x2_t*)src;
                wv[m][0] = v[0];
                wv[m][1] = v[1];
            }
            s[m] = bf16_to_f32(bs[m][grp]) * unit_inv;
            bz[m] = bf16_to_f32(bb[m][grp]);
        }
        for (int q = tid; q < MT * (KC / 8); q += 256) {
            const int row = q / (KC / 8), c8 = q % (KC / 8);
            const u32x4_t v = *(const u32x4_t*)(A + (size_t)s_row[row] * lda + c * KC + c8 * 8);
            *(u32x4_t*)(sA + row * LDA + c8 * 8) = v;
        }
        __syncthreads();
#pragma unroll
        for (int j = 0; j < W; ++j) {
            bf16x8_t bw[NMAT];
#pragma unroll
            for (int m = 0; m < NMAT; ++m) bw[m] = dequant_word(wv[m][j], s[m], bz[m]);
#pragma unroll
            for (int mi = 0; mi < MSUB; ++mi) {
                const bf16x8_t a = *(const bf16x8_t*)(sA + (mi * 16 + nl) * LDA + 8 * (g * W + j));
#pragma unroll
                for (int m = 0; m < NMAT; ++m) acc[m][mi] = mfma_16x16x32(a, bw[m], acc[m][mi]);
            }
        }
        __syncthreads();
    }

#pragma unroll
    for (int mi = 0; mi < MSUB; ++mi) {
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const int row = mi * 16 + 4 * g + i;
            if (row < nr) {
                float v;
                if constexpr (NMAT == 2) v = silu_f32(acc[0][mi][i]) * acc[1][mi][i];
                else v = acc[0][mi][i];
                out[(size_t)(r0 + row) * N + n] = __builtin_bit_cast(uint16_t, (__bf16)v);
            }
        }
    }
}

size_t gemm_ws_layout(int T, int I, int I_sh, int k, size_t* off_h, size_t* off_hsh) {
    size_t o = 0;
    *off_h = o;
    o += align_up((size_t)T * k * I * sizeof(uint16_t), 256);
    *off_hsh = o;
    o += align_up((size_t)T * I_sh * sizeof(uint16_t), 256);
    return o;
}

static int pick_kc(int K, int K2) {
    for (int kc = 256; kc >= 64; kc >>= 1)
        if (K % kc == 0 && (K2 == 0 || K2 % kc == 0)) return kc;
    return 0;
}

template <int NMAT, int MT>
static void launch_mt(const GroupedArgs& a, int kc, dim3 grid, hipStream_t stream) {
    if (kc == 256) grouped_q4_kernel<NMAT, MT, 256><<<grid, 256, 0, stream>>>(a);
    else if (kc == 128) grouped_q4_kernel<NMAT, MT, 128><<<grid, 256, 0, stream>>>(a);
    else grouped_q4_kernel<NMAT, MT, 64><<<grid, 256, 0, stream>>>(a);
}

template <int NMAT>
static void launch_grouped(const GroupedArgs& a, int mt, int kc, dim3 grid, hipStream_t stream) {
    if (mt == 16) launch_mt<NMAT, 16>(a, kc, grid, stream);
    else if (mt == 32) launch_mt<NMAT, 32>(a, kc, grid, stream);
    else launch_mt<NMAT, 64>(a, kc, grid, stream);
}

hipError_t launch_grouped_gemm(const GemmProblem& p, void* ws, hipStream_t stream) {
    size_t off_h, off_hsh;
    gemm_ws_layout(p.T, p.I, p.I_sh, p.k, &off_h, &off_hsh);
    uint16_t* h = (uint16_t*)((char*)ws + off_h);
    uint16_t* h_sh = (uint16_t*)((char*)ws + off_hsh);
    const int mt = p.block_rows;
    const int sh_blocks = p.I_sh ? (p.T + mt - 1) / mt : 0;

    GroupedArgs a{};
    a.k = p.k;
    a.T = p.T;
    a.sorted_assign = p.r.sorted_assign;
    a.block_expert = p.r.block_expert;
    a.block_row = p.r.block_row;
    a.n_blocks = p.r.n_blocks;
    a.offsets = p.r.offsets;
    a.sh_blocks = sh_blocks;
    const dim3 grid_y(1, sh_blocks + p.max_blocks);

    // gate + up with SwiGLU: A = x (gathered), N = I, K = H
    a.a_routed = p.x;
    a.a_shared = p.x;
    a.lda_routed = a.lda_shared = p.H;
    a.gather = 1;
    a.rB[0] = p.gate;
    a.rB[1] = p.up;
    a.sB[0] = p.sh_gate;
    a.sB[1] = p.sh_up;
    a.N = p.I;
    a.K = p.H;
    a.N_sh = p.I_sh;
    a.K_sh = p.H;
    a.out_routed = h;
    a.out_shared = h_sh;
    {
        const int nmax = p.I > p.I_sh ? p.I : p.I_sh;
        const dim3 grid(nmax / 64, grid_y.y);
        launch_grouped<2>(a, mt, pick_kc(p.H, 0), grid, stream);
    }

    // down: A = h rows (contiguous), N = H, K = I
    a.a_routed = h;
    a.a_shared = h_sh;
    a.lda_routed = p.I;
    a.lda_shared = p.I_sh;
    a.gather = 0;
    a.rB[0] = p.down;
    a.sB[0] = p.sh_down;
    a.N = p.H;
    a.K = p.I;
    a.N_sh = p.I_sh ? p.H : 0;
    a.K_sh = p.I_sh;
    a.out_routed = p.expert_out;
    a.out_shared = p.shared_out;
    {
        const dim3 grid(p.H / 64, grid_y.y);
        launch_grouped<1>(a, mt, pick_kc(p.I, p.I_sh), grid, stream);
    }
    return hipGetLastError();
}

}  // namespace moeq4
