// Per-token top-k selection by one wave (shared by the routing kernels and
// the fused decode kernel).  [P1] dothoosh.com Lily article, "Model
// specification": the router scores 256 experts and keeps 8.
#pragma once

#include "moe_device.h"

namespace moeq4 {

// Up to this k the selection runs as k wave-argmax rounds, above it as a
// 32-step radix select followed by an O(k^2) ranking.
constexpr int kRoundsMaxK = 16;

// Order-preserving map of a finite float to uint32 (-0.0 folded onto +0.0).
__device__ __forceinline__ uint32_t float_key(float v) {
    const uint32_t u = __builtin_bit_cast(uint32_t, v + 0.0f);
    return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}

__device__ __forceinline__ int wave_popc_ge(uint32_t key, uint32_t th, bool valid) {
    return __popcll(__ballot(valid && key >= th));
}

// Largest key over the wave, returned uniform.  DPP: row_shr 1, 2, 4, 8 leave
// each row's maximum in its lane 15; row_bcast 15 and 31 carry those into
// lane 63.  A lane whose source lies outside the wave or its row reads 0
// (bound_ctrl), which max ignores (keys are unsigned), and extra rows taking
// part in the broadcasts only take a max over windows that overlap: max is
// idempotent, so every lane still holds a max of some lanes and lane 63 the
// max of all.  The form lets the compiler fold each move into its max
// (v_max_u32 with a DPP source), one instruction per step.
__device__ __forceinline__ uint32_t wave_max_u32(uint32_t v) {
#define MOE_DPP_MAX(ctrl)                                                                 \
    v = __builtin_elementwise_max(                                                        \
        v, (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, ctrl, 0xf, 0xf, true))
    MOE_DPP_MAX(0x111);   // row_shr:1
    MOE_DPP_MAX(0x112);   // row_shr:2
    MOE_DPP_MAX(0x114);   // row_shr:4
    MOE_DPP_MAX(0x118);   // row_shr:8
    MOE_DPP_MAX(0x142);   // row_bcast:15
    MOE_DPP_MAX(0x143);   // row_bcast:31
#undef MOE_DPP_MAX
    return __builtin_amdgcn_readlane(v, 63);
}

// Inverse of float_key.
__device__ __forceinline__ float key_float(uint32_t key) {
    return __builtin_bit_cast(float, (key & 0x80000000u) ? (key & 0x7FFFFFFFu) : ~key);
}

// k rounds of "largest remaining key, lowest expert index among equals": the
// rounds produce the slots in order (value descending, index ascending), and
// the renormalised softmax weights come from the k chosen values.  Lane l
// holds experts l*EPL .. l*EPL+EPL-1; used or absent experts carry key 0.
// Costs about k * (3 EPL + 25) VALU operations, so it is used for small k.
template <int EPL>
__device__ __forceinline__ void topk_rounds(uint32_t (&key)[EPL], int k, int32_t* out_idx,
                                            float* out_w, int* lds_idx) {
    const int lane = __lane_id();
    int my_e = 0;
    float my_x = 0.0f, v0 = 0.0f, sum = 0.0f;
    for (int r = 0; r < k; ++r) {
        uint32_t bk = key[0];
        int bj = 0;
#pragma unroll
        for (int j = 1; j < EPL; ++j) {
            const bool gt = key[j] > bk;   // strict: the lower index wins a tie
            bk = gt ? key[j] : bk;
            bj = gt ? j : bj;
        }
        const uint32_t m = wave_max_u32(bk);
        const int w = __builtin_ctzll(__ballot(bk == m));          // lowest lane holding m
        const int jw = __builtin_amdgcn_readlane(bj, w);
        const float val = key_float(m);
        if (r == 0) v0 = val;
        const float x = __expf(val - v0);
        sum += x;
        if (lane == r) {
            my_e = w * EPL + jw;
            my_x = x;
        }
#pragma unroll
        for (int j = 0; j < EPL; ++j) key[j] = (lane == w && j == jw) ? 0u : key[j];
    }
    if (lane < k) {
        out_idx[lane] = my_e;
        out_w[lane] = my_x * (1.0f / sum);
        if (lds_idx) lds_idx[lane] = my_e;
    }
    __builtin_amdgcn_wave_barrier();
}

// Top-k of one token's E logits by one wave.  Lane l holds experts
// l*EPL .. l*EPL+EPL-1.  s_key/s_e/s_v: this wave's LDS scratch of k entries
// (used when k > kRoundsMaxK).  Always inlined: as an out-of-line call (which
// the compiler chose for some EPL) it spilled registers to scratch and took
// about 0.75 us per token.
template <int EPL>
__device__ __forceinline__ void topk_token(const float* __restrict__ row, int E, int k, int32_t* out_idx,
                           float* out_w, uint32_t* s_key, int* s_e, float* s_v,
                           int* lds_idx = nullptr) {
    const int lane = __lane_id();
    float v[EPL];
    uint32_t key[EPL];
    bool ok[EPL];
#pragma unroll
    for (int j = 0; j < EPL; ++j) {
        const int e = lane * EPL + j;
        ok[j] = e < E;
        v[j] = ok[j] ? row[e] : 0.0f;
        key[j] = ok[j] ? float_key(v[j]) : 0u;
    }
    if (k <= kRoundsMaxK) {
        topk_rounds<EPL>(key, k, out_idx, out_w, lds_idx);
        return;
    }
    // radix select: largest th with count(key >= th) >= k
    uint32_t th = 0;
    bool exact = false;
    for (int b = 31; b >= 0; --b) {
        const uint32_t cand = th | (1u << b);
        int c = 0;
#pragma unroll
        for (int j = 0; j < EPL; ++j) c += wave_popc_ge(key[j], cand, ok[j]);
        if (c >= k) {
            th = cand;
            if (c == k) {
                exact = true;
                break;
            }
        }
    }
    // selection mask (per element) and its position in expert order
    bool sel[EPL];
    if (exact) {
#pragma unroll
        for (int j = 0; j < EPL; ++j) sel[j] = ok[j] && key[j] >= th;
    } else {
        int gt = 0;
#pragma unroll
        for (int j = 0; j < EPL; ++j) gt += __popcll(__ballot(ok[j] && key[j] > th));
        const int need = k - gt;
        const uint64_t lt = lanemask_lt();
        int below = 0;   // ties held by lower lanes
        uint64_t tb[EPL];
#pragma unroll
        for (int j = 0; j < EPL; ++j) {
            tb[j] = __ballot(ok[j] && key[j] == th);
            below += __popcll(tb[j] & lt);
        }
        int own = 0;
#pragma unroll
        for (int j = 0; j < EPL; ++j) {
            const bool tie = ok[j] && key[j] == th;
            sel[j] = (ok[j] && key[j] > th) || (tie && below + own < need);
            own += tie ? 1 : 0;
        }
    }
    // compact the k chosen into LDS in expert order
    {
        const uint64_t lt = lanemask_lt();
        int pos = 0;
        uint64_t sb[EPL];
#pragma unroll
        for (int j = 0; j < EPL; ++j) {
            sb[j] = __ballot(sel[j]);
            pos += __popcll(sb[j] & lt);
        }
#pragma unroll
        for (int j = 0; j < EPL; ++j) {
            if (sel[j]) {
                s_key[pos] = key[j];
                s_e[pos] = lane * EPL + j;
                s_v[pos] = v[j];
                ++pos;
            }
        }
    }
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    // slot of each chosen = number of chosen ahead of it (value desc, index asc);
    // entries are in ascending expert order, so "index asc" = position order
    float vmax = -__builtin_huge_valf();
    for (int p = lane; p < k; p += WAVE) vmax = fmaxf(vmax, s_v[p]);
#pragma unroll
    for (int off = WAVE / 2; off >= 1; off >>= 1) vmax = fmaxf(vmax, shfl_xor(vmax, off));
    float part = 0.0f;
    for (int p = lane; p < k; p += WAVE) part += __expf(s_v[p] - vmax);
#pragma unroll
    for (int off = WAVE / 2; off >= 1; off >>= 1) part += shfl_xor(part, off);
    const float inv = 1.0f / part;
    for (int p = lane; p < k; p += WAVE) {
        const uint32_t kp = s_key[p];
        int slot = 0;
        for (int q = 0; q < k; ++q) {
            const uint32_t kq = s_key[q];
            slot += (kq > kp || (kq == kp && q < p)) ? 1 : 0;
        }
        out_idx[slot] = s_e[p];
        out_w[slot] = __expf(s_v[p] - vmax) * inv;
        if (lds_idx) lds_idx[slot] = s_e[p];
    }
    __builtin_amdgcn_wave_barrier();
}

}  // namespace moeq4
