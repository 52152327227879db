// Batch-1 decode of the MoE layer: two ordinary launches per token, no host
// synchronisation and no grid-wide barrier.
//
// Decode is bound by bytes moved, not by compute ([P3] droneth.or.th,
// "Decode is limited by bandwidth more than by compute"), and the engine
// removes per-token host round trips and fuses kernel chains ([P1]
// dothoosh.com Lily article, "Decode optimizations", kernel-fusion bullet).
//
//   decode_gateup_kernel: every workgroup selects the token's top-k from the
//     logits itself (the same deterministic selection as moe_route; workgroup
//     0 also publishes it), then its waves stream gate/up weight rows of the
//     k chosen experts and the shared expert, kGuRows row pairs per wave at a
//     time, and write h = bf16(silu(g) * u).
//   decode_down_kernel: each workgroup owns 4 output columns; its 8 waves
//     split the experts, stream those experts' down-projection rows for the
//     4 columns, and weight each expert's dot with topk_w (shared expert:
//     weight 1); the wave partials are summed in a fixed order, y = bf16.
//
// The weights are 4-bit groupwise affine, w = q * s + b per 64 weights ([P1]
// "Prefill optimizations", fused-dequantization bullet; [P3] "A big model
// that touches only part of its weights per token").  The pages expand them
// to bf16 because the tensor units take bf16; a batch-1 GEMV does not use the
// tensor units, and each weight row is read exactly once, so here the
// per-weight VALU work is what competes with HBM.  Each dot is therefore
// taken in its exact affine form per group, sum x (q s + b) =
// s sum q x + b sum x, in fp32: the activations are widened once per pass
// and shared by every row the wave streams, so a weight costs about two VALU
// operations (nibble to float, one FMA).  The result differs from a product
// with bf16-rounded weights only in rounding.
#include "moe_device.h"
#include "moe_launch.h"
#include "moe_topk.h"

namespace moeq4 {

// Gate/up shape: waves per workgroup x row pairs per wave.  8 x 1 (576
// workgroups, one top-k per 8 rows) measured fastest with the shared rows last:
// 11.9 us per token against 12.0 for 4 x 1, 12.3 for 4 x 2, 12.5 for 8 x 2,
// 12.6 for 12 x 1, 13.4 for 2 x 1 and 14.9 for 16 x 1.
#ifndef MOE_DEC_GU_WAVES
#define MOE_DEC_GU_WAVES 8
#endif
constexpr int kDecWaves = MOE_DEC_GU_WAVES;
constexpr int kDecThreads = kDecWaves * WAVE;
constexpr int kDecMaxK = 64;
#ifndef MOE_DEC_GU_ROWS
#define MOE_DEC_GU_ROWS 1
#endif
#ifndef MOE_DEC_DN_EXP
#define MOE_DEC_DN_EXP 1
#endif
constexpr int kGuRows = MOE_DEC_GU_ROWS;   // gate/up row pairs one wave streams together
constexpr int kDnExp = MOE_DEC_DN_EXP;     // experts whose down rows one wave loads together
constexpr int kDnCols = 4;    // output columns per down workgroup (16 lanes each)
#ifndef MOE_DEC_DN_WAVES
#define MOE_DEC_DN_WAVES 9
#endif
// waves of a down workgroup; they split the k + 1 experts, one each at k = 8
// (with the 8 x 1 gate/up shape: 9 and 12 waves 12.2 us per token cold, 8 waves
// 12.4, 4 waves 13.2, 16 waves 13.8)
constexpr int kDnWaves = MOE_DEC_DN_WAVES;
constexpr int kDnThreads = kDnWaves * WAVE;

// q * 2^-9 for the 8 codes of a packed word, in code order (low nibble first).
__device__ __forceinline__ void codes_unit(uint32_t w, float (&q)[8]) {
    const uint32_t lo = w & 0x0F0F0F0Fu;         // codes 0, 2, 4, 6
    const uint32_t hi = (w >> 4) & 0x0F0F0F0Fu;  // codes 1, 3, 5, 7
    const f32x2_t q02 = __builtin_amdgcn_cvt_pk_f32_fp8((int)lo, false);
    const f32x2_t q46 = __builtin_amdgcn_cvt_pk_f32_fp8((int)lo, true);
    const f32x2_t q13 = __builtin_amdgcn_cvt_pk_f32_fp8((int)hi, false);
    const f32x2_t q57 = __builtin_amdgcn_cvt_pk_f32_fp8((int)hi, true);
    q[0] = q02[0]; q[1] = q13[0]; q[2] = q02[1]; q[3] = q13[1];
    q[4] = q46[0]; q[5] = q57[0]; q[6] = q46[1]; q[7] = q57[1];
}

// 32 bf16 activations (4 x 16 B) widened to fp32 (exact), and their sum.
__device__ __forceinline__ float widen32(const u32x4_t (&v)[4], float (&f)[32]) {
    float s = 0.0f;
#pragma unroll
    for (int i = 0; i < 16; ++i) {
        const uint32_t w = v[i / 4][i % 4];
        f[2 * i] = __builtin_bit_cast(float, w << 16);
        f[2 * i + 1] = __builtin_bit_cast(float, w & 0xFFFF0000u);
        s += f[2 * i] + f[2 * i + 1];
    }
    return s;
}

// sum_i (q_i * 2^-9) * f_i over the 32 codes of 4 packed words.
__device__ __forceinline__ float qdot32(const u32x4_t& w, const float (&f)[32]) {
    float a = 0.0f;
#pragma unroll
    for (int j = 0; j < 4; ++j) {
        float q[8];
        codes_unit(w[j], q);
#pragma unroll
        for (int i = 0; i < 8; ++i) a = __builtin_fmaf(q[i], f[8 * j + i], a);
    }
    return a;
}

// One butterfly step over lane distance M for CNT values, then the next ones
// (compile-time recursion, so v stays in registers; a run-time loop here
// would index v dynamically and move it to shared memory).
template <int CNT, int M, int NV>
__device__ __forceinline__ void reduce_steps(float (&v)[NV], int lane) {
    if constexpr (CNT > 1) {
        const bool upper = (lane & M) != 0;
#pragma unroll
        for (int i = 0; i < CNT / 2; ++i) {
            const float keep = upper ? v[i + CNT / 2] : v[i];
            const float send = upper ? v[i] : v[i + CNT / 2];
            v[i] = keep + shfl_xor(send, M);
        }
        reduce_steps<CNT / 2, M / 2>(v, lane);
    }
}

// Butterfly reduction of NV values over the wave.  Afterwards every lane
// holds the full sum of one value: the top log2(NV) lane bits, read from
// bit 5 down, are the binary digits of that value's index (most significant
// first).
template <int NV>
__device__ __forceinline__ float wave_reduce_multi(float (&v)[NV], int lane) {
    static_assert(NV >= 1 && NV <= WAVE && (NV & (NV - 1)) == 0, "a power of two up to 64");
    reduce_steps<NV, WAVE / 2>(v, lane);
    float s = v[0];
#pragma unroll
    for (int m = WAVE / 2 / NV; m >= 1; m /= 2) s += shfl_xor(s, m);
    return s;
}

// T = 1 routing arrays from the chosen experts (workgroup-uniform call).
__device__ void write_routing_t1(const DecodeArgs& p, const int* s_idx, const float* s_w,
                                 int tid) {
    const int k = p.k;
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

// SB: gate and up carry packed scale|bias words (MOE_Q4_LAYOUT_TILES_SB), word
// ((row / 64) * G + group) * 64 + row % 64 of the matrix set.
template <int EPL, bool SB>
__global__ __launch_bounds__(kDecThreads) void decode_gateup_kernel(DecodeArgs p) {
    __shared__ int s_idx[kDecMaxK];
    __shared__ float s_w[kDecMaxK];
    __shared__ uint32_t s_scr[3 * kDecMaxK];
    const int tid = threadIdx.x, lane = tid % WAVE;
    // wave-uniform from here on, so row addresses stay in scalar registers
    const int wave = __builtin_amdgcn_readfirstlane(tid / WAVE);
    const int k = p.k, H = p.H, I = p.I, I_sh = p.I_sh;

    // Tasks are the k selected experts' rows (expert j's rows after expert
    // j - 1's), then the shared expert's rows, whose workgroups need no top-k
    // and start streaming at once.  They come last in the grid because the
    // workgroups that share a CU with others finish in the order they were
    // placed there, and the shared rows, streaming from the start, make the
    // best last ones.  One pass of the grid covers every task, so this
    // workgroup's rows are tasks [8b, 8b + 8) (workgroup 0 always selects, to
    // publish the selection).
    const int routed_tasks = k * I;
    const bool need_topk =
        blockIdx.x == 0 || (int)blockIdx.x * kDecWaves * kGuRows < routed_tasks;
    if (wave == 0 && need_topk)
        topk_token<EPL>(p.logits, p.E, k, s_idx, s_w, s_scr, (int*)(s_scr + k),
                        (float*)(s_scr + 2 * k), nullptr);
    __syncthreads();
    if (blockIdx.x == 0) {
        if (tid < k) {
            p.sel_idx[tid] = s_idx[tid];
            p.sel_w[tid] = s_w[tid];
        }
        if (p.write_routing) write_routing_t1(p, s_idx, s_w, tid);
    }

    const int ldh = I > I_sh ? I : I_sh;
    const int n_tasks = routed_tasks + I_sh;
    const float unit_inv = 1.0f / fp8_unit();
    const int stride = gridDim.x * kDecWaves * kGuRows;
    for (int t0 = (blockIdx.x * kDecWaves + wave) * kGuRows; t0 < n_tasks; t0 += stride) {
        const uint32_t* gc[kGuRows];   // expert's code matrix (row n_r is addressed per layout)
        const uint32_t* uc[kGuRows];
        const uint16_t *gs[kGuRows], *gb[kGuRows], *us[kGuRows], *ub[kGuRows];
        const uint32_t *gsb[kGuRows], *usb[kGuRows];   // SB: the row's word of group 0
        int hidx[kGuRows], nrow[kGuRows];
#pragma unroll
        for (int r = 0; r < kGuRows; ++r) {
            const int t = t0 + r < n_tasks ? t0 + r : n_tasks - 1;   // tail: re-read a valid row
            const bool sh = t >= routed_tasks;
            const int j = sh ? k : t / I;
            const int n = sh ? t - routed_tasks : t - j * I;
            const size_t row = sh ? (size_t)n : (size_t)__builtin_amdgcn_readfirstlane(s_idx[j]) * I + n;
            const QMatDev& g = sh ? p.sh_gate : p.gate;
            const QMatDev& u = sh ? p.sh_up : p.up;
            const size_t ebase = (row - n) * (H / 8);   // first word of the expert's matrix
            gc[r] = g.codes + ebase;
            uc[r] = u.codes + ebase;
            nrow[r] = n;
            gs[r] = g.scales + row * (H / 64);
            gb[r] = g.biases + row * (H / 64);
            us[r] = u.scales + row * (H / 64);
            ub[r] = u.biases + row * (H / 64);
            const size_t sbw = (row / 64) * (size_t)(H / 64) * 64 + row % 64;
            gsb[r] = (const uint32_t*)g.scales + sbw;
            usb[r] = (const uint32_t*)u.scales + sbw;
            hidx[r] = t0 + r < n_tasks ? j * ldh + n : -1;
        }
        float acc[2 * kGuRows];
#pragma unroll
        for (int i = 0; i < 2 * kGuRows; ++i) acc[i] = 0.0f;
        for (int kb = lane * 32; kb < H; kb += WAVE * 32) {
            u32x4_t xv[4];
#pragma unroll
            for (int q = 0; q < 4; ++q) xv[q] = *(const u32x4_t*)(p.x + kb + 8 * q);
            u32x4_t gw[kGuRows], uw[kGuRows];
            float sg[kGuRows], bg[kGuRows], su[kGuRows], bu[kGuRows];
            const int grp = kb / 64;
#pragma unroll
            for (int r = 0; r < kGuRows; ++r) {
                const uint32_t wo = code_word(p.gate.layout, nrow[r], kb / 8, H);
                gw[r] = *(const u32x4_t*)(gc[r] + wo);
                uw[r] = *(const u32x4_t*)(uc[r] + wo);
                if constexpr (SB) {
                    const uint32_t wg = gsb[r][grp * 64], wu = usb[r][grp * 64];
                    sg[r] = bf16_to_f32((uint16_t)(wg & 0xFFFFu));
                    bg[r] = bf16_to_f32((uint16_t)(wg >> 16));
                    su[r] = bf16_to_f32((uint16_t)(wu & 0xFFFFu));
                    bu[r] = bf16_to_f32((uint16_t)(wu >> 16));
                } else {
                    sg[r] = bf16_to_f32(gs[r][grp]);
                    bg[r] = bf16_to_f32(gb[r][grp]);
                    su[r] = bf16_to_f32(us[r][grp]);
                    bu[r] = bf16_to_f32(ub[r][grp]);
                }
            }
            // every load of the pass is issued before the first wait (the scheduler
            // would otherwise interleave them with the math, one row per round trip)
            __builtin_amdgcn_sched_barrier(0);
            float xf[32];
            const float sx = widen32(xv, xf);
#pragma unroll
            for (int r = 0; r < kGuRows; ++r) {
                acc[r] = __builtin_fmaf(sg[r] * unit_inv, qdot32(gw[r], xf),
                                        __builtin_fmaf(bg[r], sx, acc[r]));
                acc[kGuRows + r] = __builtin_fmaf(su[r] * unit_inv, qdot32(uw[r], xf),
                                                  __builtin_fmaf(bu[r], sx, acc[kGuRows + r]));
            }
        }
        // value i (g of row i, then u of row i - kGuRows) ends in lanes
        // [i * kLanesPerVal, (i + 1) * kLanesPerVal): lane l < 32 holds g of row
        // l / kLanesPerVal and lane l + 32 holds u of that row
        constexpr int kLanesPerVal = WAVE / (2 * kGuRows);
        const float gsum = wave_reduce_multi<2 * kGuRows>(acc, lane);
        const float usum = shfl_xor(gsum, WAVE / 2);
        const int r = lane / kLanesPerVal;
        if (lane < WAVE / 2 && lane % kLanesPerVal == 0) {
            int hi = hidx[0];
#pragma unroll
            for (int q = 1; q < kGuRows; ++q) hi = r == q ? hidx[q] : hi;
            if (hi >= 0) p.h[hi] = __builtin_bit_cast(uint16_t, (__bf16)(silu_f32(gsum) * usum));
        }
    }
}

__global__ __launch_bounds__(kDnThreads) void decode_down_kernel(DecodeArgs p) {
    __shared__ float s_part[kDnWaves][kDnCols];
    const int tid = threadIdx.x, lane = tid % WAVE;
    const int wave = __builtin_amdgcn_readfirstlane(tid / WAVE);
    const int k = p.k, H = p.H, I = p.I, I_sh = p.I_sh;
    const int ldh = I > I_sh ? I : I_sh;
    const int nexp = k + (I_sh ? 1 : 0);    // slot k is the shared expert
    const int c = blockIdx.x * kDnCols + lane / 16;
    const int kl = (lane % 16) * 32;
    const float unit_inv = 1.0f / fp8_unit();
    float acc = 0.0f;
    for (int j0 = wave; j0 < nexp; j0 += kDnWaves * kDnExp) {
        const uint32_t* dc[kDnExp];
        const uint16_t *ds[kDnExp], *db[kDnExp];
        const uint16_t* hp[kDnExp];
        float wj[kDnExp];
        int N[kDnExp];
#pragma unroll
        for (int i = 0; i < kDnExp; ++i) {
            const int j = j0 + i * kDnWaves;
            const bool on = j < nexp;
            const bool sh = j == k;
            const int e = on && !sh ? p.sel_idx[j] : 0;
            const QMatDev& d = sh ? p.sh_down : p.down;
            N[i] = !on ? 0 : sh ? I_sh : I;
            const int Nr = N[i] ? N[i] : 64;
            const size_t row = (size_t)e * H + c;
            dc[i] = d.codes + (size_t)e * H * (Nr / 8);   // expert's code matrix; row c per layout
            ds[i] = d.scales + row * (Nr / 64);
            db[i] = d.biases + row * (Nr / 64);
            hp[i] = p.h + (size_t)(on ? j : 0) * ldh;
            wj[i] = on ? (sh ? 1.0f : p.sel_w[j]) : 0.0f;
        }
        for (int kb = kl; kb < ldh; kb += 16 * 32) {
            u32x4_t cw[kDnExp], hv[kDnExp][4];
            float s[kDnExp], b[kDnExp];
#pragma unroll
            for (int i = 0; i < kDnExp; ++i) {
                if (kb < N[i]) {
                    cw[i] = *(const u32x4_t*)(dc[i] + code_word(p.down.layout, c, kb / 8, N[i]));
                    s[i] = bf16_to_f32(ds[i][kb / 64]);
                    b[i] = bf16_to_f32(db[i][kb / 64]);
#pragma unroll
                    for (int q = 0; q < 4; ++q) hv[i][q] = *(const u32x4_t*)(hp[i] + kb + 8 * q);
                } else {
                    cw[i] = u32x4_t{0, 0, 0, 0};
                    s[i] = 0.0f;
                    b[i] = 0.0f;
#pragma unroll
                    for (int q = 0; q < 4; ++q) hv[i][q] = u32x4_t{0, 0, 0, 0};
                }
            }
            __builtin_amdgcn_sched_barrier(0);
#pragma unroll
            for (int i = 0; i < kDnExp; ++i) {
                float hf[32];
                const float hs = widen32(hv[i], hf);
                const float part = __builtin_fmaf(s[i] * unit_inv, qdot32(cw[i], hf), b[i] * hs);
                acc = __builtin_fmaf(wj[i], part, acc);
            }
        }
    }
#pragma unroll
    for (int off = 8; off >= 1; off >>= 1) acc += shfl_xor(acc, off);
    if ((lane & 15) == 0) s_part[wave][lane / 16] = acc;
    __syncthreads();
    if (tid < kDnCols) {
        float y = 0.0f;
#pragma unroll
        for (int w = 0; w < kDnWaves; ++w) y += s_part[w][tid];
        p.y[blockIdx.x * kDnCols + tid] = __builtin_bit_cast(uint16_t, (__bf16)y);
    }
}

DecodeWs decode_ws_layout(int H, int I, int I_sh, int k) {
    (void)H;
    DecodeWs w{};
    const int ldh = I > I_sh ? I : I_sh;
    size_t o = 0;
    auto take = [&](size_t bytes) {
        const size_t at = o;
        o += align_up(bytes, 256);
        return at;
    };
    w.h = take((size_t)(k + 1) * ldh * sizeof(uint16_t));
    w.sel_idx = take(kDecMaxK * sizeof(int32_t));
    w.sel_w = take(kDecMaxK * sizeof(float));
    w.total = o;
    return w;
}

void decode_launch_shapes(int H, int I, int I_sh, int k, int* grid1, int* threads1, int* grid2,
                          int* threads2) {
    const int chunks = (I_sh + k * I + kGuRows - 1) / kGuRows;
    *grid1 = (chunks + kDecWaves - 1) / kDecWaves;
    *threads1 = kDecThreads;
    *grid2 = H / kDnCols;
    *threads2 = kDnThreads;
}

template <int EPL>
static void launch_gateup_epl(const DecodeArgs& args, int g1, int t1, hipStream_t stream) {
    if (args.gate.layout == 2)
        hipLaunchKernelGGL((decode_gateup_kernel<EPL, true>), dim3(g1), dim3(t1), 0, stream, args);
    else
        hipLaunchKernelGGL((decode_gateup_kernel<EPL, false>), dim3(g1), dim3(t1), 0, stream, args);
}

hipError_t launch_decode(const DecodeArgs& args, hipStream_t stream) {
    int g1, t1, g2, t2;
    decode_launch_shapes(args.H, args.I, args.I_sh, args.k, &g1, &t1, &g2, &t2);
    const int epl = (args.E + WAVE - 1) / WAVE;
    if (epl <= 1) launch_gateup_epl<1>(args, g1, t1, stream);
    else if (epl <= 2) launch_gateup_epl<2>(args, g1, t1, stream);
    else if (epl <= 4) launch_gateup_epl<4>(args, g1, t1, stream);
    else if (epl <= 8) launch_gateup_epl<8>(args, g1, t1, stream);
    else launch_gateup_epl<16>(args, g1, t1, stream);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    hipLaunchKernelGGL(decode_down_kernel, dim3(g2), dim3(t2), 0, stream, args);
    return hipGetLastError();
}

}  // namespace moeq4
