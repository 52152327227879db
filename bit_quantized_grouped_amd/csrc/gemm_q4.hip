// Grouped expert GEMM with the 4-bit dequantization fused into the tiles
// ([P1] dothoosh.com Lily article, "Prefill optimizations", fused
// dequantization bullet; [P3] droneth.or.th, "A big model that touches only
// part of its weights per token": weights are rebuilt tile by tile inside the
// grouped GEMM as bf16 and accumulated in FP32; expanded weights never reach
// memory).
//
// One kernel template serves both projections:
//   NMAT = 2  gate and up over the same output columns, SwiGLU epilogue
//             h = silu(g) * u -> bf16 h  (A = x rows gathered by token)
//   NMAT = 1  down projection -> bf16 expert_out / shared_out
//             (A = h rows, contiguous in sorted-row order)
// Work item = one row block of the block map (MT rows of one expert) x
// COLS = 4 waves x NSUB x 16 output columns.  The shared expert is an extra
// dense group over all tokens, as the first sh_blocks row blocks.
//
// Data path per K-chunk of KC:
//   A: the block's MT rows x KC bf16 are fetched DEPTH-1 chunks ahead into
//      registers, then staged in LDS (double-buffered, row stride KC+8 so
//      ds_read_b128 is conflict free) and read by every wave.  With packed
//      scale|bias words and 128-K chunks they go straight from memory into a
//      3-tile LDS ring instead (buffer loads with the LDS flag, dense rows
//      with XOR-swizzled 16-byte pieces), two chunks ahead;
//   B: each lane streams KC/32 consecutive code words of each of its weight
//      rows straight from HBM into registers with buffer loads (4 lanes
//      cover a row's KC/2 bytes contiguously; the chunk and subtile offsets
//      ride in the scalar offset, so no per-load address arithmetic),
//      DEPTH-1 chunks ahead of the math, with the row's scale|bias word of
//      the chunk's group when the words are packed (else the scales and
//      biases of the tile's rows sit in LDS).  Each word (8 weights) is dequantized
//      in registers to bf16 and fed to v_mfma_f32_16x16x32_bf16.  A lane's 8
//      weights are the 8 consecutive k of its word, so both operands use the
//      natural K order inside each MFMA.
//   Epilogue: accumulators -> bf16 tile in LDS -> 16-byte row stores.
#include "moe_device.h"
#include "moe_launch.h"

// Tile shape per projection: NSUB 16-column subtiles per wave, the largest
// K-chunk (a divisor of K is used), and the number of chunks of code words in
// flight per wave (register pipeline depth).
#ifndef MOE_GU_WAVES
#define MOE_GU_WAVES 4
#endif
#ifndef MOE_GU_NSUB
#define MOE_GU_NSUB 1
#endif
#ifndef MOE_GU_KC
#define MOE_GU_KC 128
#endif
#ifndef MOE_GU_DEPTH
#define MOE_GU_DEPTH 4
#endif
// With packed scale|bias words the workgroup needs only the A tiles in LDS;
// a 2-deep ring then keeps the registers low enough for 6 waves per SIMD.
#ifndef MOE_GU_SB_DEPTH
#define MOE_GU_SB_DEPTH 2
#endif
#ifndef MOE_DN_WAVES
#define MOE_DN_WAVES 8
#endif
#ifndef MOE_DN_NSUB
#define MOE_DN_NSUB 1
#endif
#ifndef MOE_DN_KC
#define MOE_DN_KC 128
#endif
#ifndef MOE_DN_DEPTH
#define MOE_DN_DEPTH 4
#endif
// Resident workgroups per CU are capped by reserving LDS (0 = no cap): with
// equal work items, the item count over resident slots sets how full the
// last dispatch round is.
#ifndef MOE_GU_WG_PER_CU
#define MOE_GU_WG_PER_CU 0
#endif
#ifndef MOE_DN_WG_PER_CU
#define MOE_DN_WG_PER_CU 0
#endif

namespace moeq4 {

typedef __amdgpu_buffer_rsrc_t rsrc_t;

// Raw buffer resource over [base, base + bytes); loads past the end return 0.
__device__ __forceinline__ rsrc_t make_rsrc(const void* base, uint32_t bytes) {
    return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0, bytes, 0x00020000);
}

struct GroupedArgs {
    const uint16_t* a_routed;
    const uint16_t* a_shared;
    int lda_routed, lda_shared;
    int rows_routed, rows_shared;   // rows of the A arrays (bounds of the A resources)
    int gather;                     // routed A rows: 1 -> token sorted_assign[row]/k, 0 -> row
    int k;
    int T;
    const int32_t* sorted_assign;
    const int32_t* block_expert;
    const int32_t* block_row;
    const int32_t* n_blocks;
    const int32_t* offsets;
    int sh_blocks;
    QMatDev rB[2];
    const uint16_t* rW[2];          // bf16-weight mode: routed weights [E, N, K]
    const uint16_t* sW[2];          // bf16-weight mode: shared weights [1, N_sh, K_sh]
    QMatDev sB[2];
    int N, K, N_sh, K_sh;
    int n_tiles;                    // column tiles per row block (of the wider of N, N_sh)
    uint16_t* out_routed;
    uint16_t* out_shared;
};

// Work item -> workgroup.  Workgroups are dispatched round-robin over the
// 8 XCDs (each with its own L2), so workgroup L runs on XCD L % 8.  The
// valid items (a count known only on the device) are split into 8
// contiguous ranges, one per XCD: the column tiles of one row block, and
// consecutive blocks of one expert, then share an L2.
constexpr int kXcds = 8;

// A compile-time flag passed as a value (to instantiate a lambda body twice).
template <bool B>
struct BoolTag {
    static constexpr bool value = B;
};

// One K-chunk of a lane's B operand: W code words per weight row (4-bit
// weights), or, in the bf16-weight mode (BF), W x 8 bf16 weights per row.
template <int NMAT, int NSUB, int W, bool BF = false>
struct BChunk {
    u32x4_t w[NMAT][NSUB][W / 4 > 0 ? W / 4 : 1];
    u32x2_t w2[NMAT][NSUB];           // used when W == 2
    u32x4_t wb[NMAT][NSUB][BF ? W : 1];
    uint32_t sb[NMAT][NSUB];          // packed scale|bias word of the lane's row and group (SB)
};

template <int NMAT, int NSUB, int KC>
struct Streams {
    rsrc_t codes[NMAT];
    int voff_c;                       // per-lane byte offset (row, lane group)
    int sub_c;                        // byte offset of subtile s is s * sub_c (row-major, bf16)
    int sub_off[NSUB];                // byte offset of subtile s (tile-packed codes)
    int chunk_c;                      // byte step per K-chunk in codes
    bool tiles;                       // codes are tile-packed
    rsrc_t sbr[NMAT];                 // packed scale|bias words (SB)
    int sb_off[NSUB];                 // per-lane byte offset of subtile s in them
    int sb_chunk;                     // byte step per K-chunk in them
};

// Chunks past the last one (pipeline run-out) are requested with kVoffOob
// added to the lane offset: such a load lies outside the buffer resource and
// returns zeros without touching memory.  Every pipeline step thus issues the
// same loads, which lets the compiler count the loads in flight across the
// loop and wait only for the chunk it is about to use (with conditional
// loads it waits for all of them once per pass over the register ring).
constexpr int kVoffOob = 0x40000000;

typedef __attribute__((address_space(3))) void* lds_ptr_t;

// 16 bytes per lane from a buffer straight into LDS: lane l writes lds + 16 l
// (lds wave-uniform).  The builtin exists only in the device pass.
__device__ __forceinline__ void buffer_load_lds16(rsrc_t r, void* lds, int voff, int soff) {
#if defined(__HIP_DEVICE_COMPILE__)
    __builtin_amdgcn_raw_ptr_buffer_load_lds(r, (lds_ptr_t)lds, 16, voff, soff, 0, 0);
#endif
}

// s_waitcnt vmcnt(n), leaving expcnt and lgkmcnt at their maxima (no wait on them).
#define MOE_WAIT_VM(n) \
    __builtin_amdgcn_s_waitcnt(((n) & 0xF) | (((n) >> 4) << 14) | (0x7 << 4) | (0xF << 8))

// Workgroup barrier without a memory fence: the caller has already waited for
// what the other waves must see (a fenced barrier would also wait for every
// load still in flight into LDS).  The signal fences keep the compiler from
// moving memory accesses across it, the scheduling barriers the scheduler.
__device__ __forceinline__ void bare_barrier() {
    __atomic_signal_fence(__ATOMIC_SEQ_CST);
    __builtin_amdgcn_sched_barrier(0);
    __builtin_amdgcn_s_barrier();
    __builtin_amdgcn_sched_barrier(0);
    __atomic_signal_fence(__ATOMIC_SEQ_CST);
}

// Cache-policy operand of a buffer load: the non-temporal hint (nt), which
// inserts the lines as the first to be evicted.
constexpr int kNonTemporal = 2;

// STREAMED: the code and scale words are requested with the non-temporal hint.
template <int NMAT, int NSUB, int KC, bool BF, bool SB, bool STREAMED = false>
__device__ __forceinline__ void load_b(BChunk<NMAT, NSUB, KC / 32, BF>& B,
                                       const Streams<NMAT, NSUB, KC>& S, int c, int voff_oob) {
    constexpr int W = KC / 32;
    constexpr int CP = STREAMED ? kNonTemporal : 0;
#pragma unroll
    for (int m = 0; m < NMAT; ++m)
#pragma unroll
        for (int s = 0; s < NSUB; ++s) {
            if constexpr (SB)
                B.sb[m][s] = __builtin_amdgcn_raw_buffer_load_b32(
                    S.sbr[m], S.sb_off[s] + voff_oob, c * S.sb_chunk, CP);
            if constexpr (BF) {   // bf16 rows: K * 2 bytes; a chunk is KC * 2 bytes of a row
                const int so_b = s * S.sub_c + c * (KC * 2);
#pragma unroll
                for (int j = 0; j < W; ++j)
                    B.wb[m][s][j] = __builtin_bit_cast(
                        u32x4_t, __builtin_amdgcn_raw_buffer_load_b128(
                                     S.codes[m], S.voff_c + voff_oob + 16 * j, so_b, 0));
                continue;
            }
            const int so_c = (S.tiles ? S.sub_off[s] : s * S.sub_c) + c * S.chunk_c;
            if constexpr (W >= 4) {
#pragma unroll
                for (int j = 0; j < W / 4; ++j)
                    B.w[m][s][j] = __builtin_bit_cast(
                        u32x4_t, __builtin_amdgcn_raw_buffer_load_b128(
                                     S.codes[m], S.voff_c + voff_oob + 16 * j, so_c, CP));
            } else {
                B.w2[m][s] = __builtin_bit_cast(
                    u32x2_t,
                    __builtin_amdgcn_raw_buffer_load_b64(S.codes[m], S.voff_c + voff_oob, so_c, CP));
            }
        }
}

template <int NMAT, int NSUB, int W, bool BF>
__device__ __forceinline__ uint32_t word_of(const BChunk<NMAT, NSUB, W, BF>& B, int m, int s, int j) {
    if constexpr (W >= 4) return B.w[m][s][j / 4][j % 4];
    else return B.w2[m][s][j];
}

// sSc / sBi: this lane's row of bf16 scales / biases in LDS (row stride GS,
// matrix stride mstride); grp = the group of the lane's words in this chunk.
// XL: the A tile is dense (row stride KC) with 16-byte piece p of row r at
// piece position p ^ (r % 16), as the direct-to-LDS x loads write it.
template <int NMAT, int MT, int KC, int NSUB, bool BF, bool SB, bool XL = false>
__device__ __forceinline__ void compute_chunk(const BChunk<NMAT, NSUB, KC / 32, BF>& B,
                                              const uint16_t* sAc, const uint16_t* sSc,
                                              const uint16_t* sBi, int GS, int mstride, int grp,
                                              float unit_inv, int nl, int g, int msub_act,
                                              f32x4_t (&acc)[NMAT][NSUB][MT / 16]) {
    constexpr int W = KC / 32;
    constexpr int LDA = KC + 8;
    float sc[NMAT][NSUB], bi[NMAT][NSUB];
#pragma unroll
    for (int m = 0; m < NMAT; ++m)
#pragma unroll
        for (int s = 0; s < NSUB; ++s) {
            if constexpr (BF) break;
            if constexpr (SB) {
                sc[m][s] = bf16_to_f32((uint16_t)(B.sb[m][s] & 0xFFFFu)) * unit_inv;
                bi[m][s] = bf16_to_f32((uint16_t)(B.sb[m][s] >> 16));
                continue;
            }
            const int at = m * mstride + s * 16 * GS + grp;
            sc[m][s] = bf16_to_f32(sSc[at]) * unit_inv;
            bi[m][s] = bf16_to_f32(sBi[at]);
        }
#pragma unroll
    for (int j = 0; j < W; ++j) {
        bf16x8_t bw[NMAT][NSUB];
#pragma unroll
        for (int m = 0; m < NMAT; ++m)
#pragma unroll
            for (int s = 0; s < NSUB; ++s)
                if constexpr (BF) bw[m][s] = __builtin_bit_cast(bf16x8_t, B.wb[m][s][j]);
                else bw[m][s] = dequant_word(word_of(B, m, s, j), sc[m][s], bi[m][s]);
#pragma unroll
        for (int mi = 0; mi < MT / 16; ++mi) {
            if (mi > 0 && mi >= msub_act) break;   // 16-row subtiles past the block's rows
            const bf16x8_t a =
                XL ? *(const bf16x8_t*)(sAc + (mi * 16 + nl) * KC + 8 * ((g * W + j) ^ nl))
                   : *(const bf16x8_t*)(sAc + (mi * 16 + nl) * LDA + 8 * (g * W + j));
#pragma unroll
            for (int m = 0; m < NMAT; ++m)
#pragma unroll
                for (int s = 0; s < NSUB; ++s)
                    acc[m][s][mi] = mfma_16x16x32(a, bw[m][s], acc[m][s][mi]);
        }
    }
}

// BF: the weights are plain bf16 [n_exp, N, K] (rW / sW), already expanded
// in memory; the unfused layout the pages compare against.
// SB: the matrices carry packed scale|bias words (MOE_Q4_LAYOUT_TILES_SB):
// each lane loads its row's word for the chunk's group with its code words,
// so the workgroup keeps no scale table in LDS and preloads nothing (the
// LDS holds only the A tiles, which lets more workgroups share a CU).
// With packed words and 128-K chunks the kernel is held to 6 waves per SIMD:
// its loop exists twice (weight words with or without the non-temporal hint),
// which the register allocator would otherwise widen past that occupancy.
template <int NMAT, int MT, int KC, int NSUB, int DEPTH, int WAVES, bool BF = false,
          bool SB = false>
__global__ __launch_bounds__(WAVES * 64)
__attribute__((amdgpu_waves_per_eu(SB && KC == 128 ? 6 : 1, 8)))
void grouped_q4_kernel(GroupedArgs p) {
    constexpr int NT = WAVES * 64;   // threads
    constexpr int W = KC / 32;       // code words per lane per chunk
    constexpr int MSUB = MT / 16;
    constexpr int LDA = KC + 8;
    constexpr int ROWS = WAVES * NSUB * 16;        // weight rows (output columns) per matrix
    constexpr int COLS = ROWS;
    constexpr int A_PIECES = MT * (KC / 8);        // 16-byte pieces of the A tile per chunk
    constexpr int APT = (A_PIECES + NT - 1) / NT;  // per thread
    // LDS: [A buffer 0][A buffer 1][scale|bias pairs]; the output tile reuses it at the end
    extern __shared__ __attribute__((aligned(16))) uint16_t smem_g[];
    __shared__ int s_row[MT];
    // XL (packed words, 128-K chunks): the x rows go straight from memory into a
    // ring of three LDS tiles, two chunks ahead of their math, with no register
    // staging; three separate arrays let the compiler tell their loads apart
    constexpr bool XL = SB && KC == 128;
    __shared__ __attribute__((aligned(16))) uint16_t sX0[XL ? MT * KC : 8];
    __shared__ __attribute__((aligned(16))) uint16_t sX1[XL ? MT * KC : 8];
    __shared__ __attribute__((aligned(16))) uint16_t sX2[XL ? MT * KC : 8];

    const int tid = threadIdx.x;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6), lane = tid & 63;
    const int nl = lane & 15, g = lane >> 4;

    // ---- work item ----
    const int n_items = (p.sh_blocks + p.n_blocks[0]) * p.n_tiles;
    const int per = (n_items + kXcds - 1) / kXcds;
    const int xcd = blockIdx.x % kXcds, seq = blockIdx.x / kXcds;
    const int item = xcd * per + seq;
    if (seq >= per || item >= n_items) return;
    const int slot = item / p.n_tiles, tile = item % p.n_tiles;
    const bool is_sh = slot < p.sh_blocks;

    int r0, nr, N, K, lda, a_rows, expert = 0;
    const uint16_t* A;
    uint16_t* out;
    if (is_sh) {
        r0 = slot * MT;
        nr = min(MT, p.T - r0);
        N = p.N_sh;
        K = p.K_sh;
        A = p.a_shared;
        lda = p.lda_shared;
        a_rows = p.rows_shared;
        out = p.out_shared;
    } else {
        const int b = slot - p.sh_blocks;
        expert = p.block_expert[b];
        r0 = p.block_row[b];
        nr = min(MT, p.offsets[expert + 1] - r0);
        N = p.N;
        K = p.K;
        A = p.a_routed;
        lda = p.lda_routed;
        a_rows = p.rows_routed;
        out = p.out_routed;
    }
    const int n_base = tile * COLS;
    if (n_base >= N) return;   // uniform per workgroup
    const int G = K / 64;      // scale groups per weight row
    const int GS = G + 8;      // padded LDS row stride (16-byte rows, conflict-free lane reads)

    uint16_t* sA = smem_g;
    uint16_t* sSc = smem_g + 2 * MT * LDA;          // [NMAT][ROWS][GS] scales
    uint16_t* sBi = sSc + NMAT * ROWS * GS;         // [NMAT][ROWS][GS] biases

    if (tid < MT) {
        const int rr = min(tid, nr - 1);   // padding rows repeat the last row; never stored
        s_row[tid] = (is_sh || !p.gather) ? r0 + rr : p.sorted_assign[r0 + rr] / p.k;
    }

    // ---- scale/bias pairs of the tile's ROWS rows, all K, into LDS ----
    // (rows are contiguous in the scale arrays: 16-byte coalesced loads;
    //  rows past N fall outside the buffer resource and read as zero)
    Streams<NMAT, NSUB, KC> S;
#pragma unroll
    for (int m = 0; m < NMAT; ++m) {
        const size_t rows0 = (size_t)expert * N;
        if constexpr (BF) {   // expanded bf16 weights: no scales
            S.codes[m] = make_rsrc((is_sh ? p.sW[m] : p.rW[m]) + rows0 * K, (uint32_t)N * K * 2);
            continue;
        }
        const QMatDev& q = is_sh ? p.sB[m] : p.rB[m];
        S.codes[m] = make_rsrc(q.codes + rows0 * (K / 8), (uint32_t)N * (K / 2));
        if constexpr (SB) {   // packed words [row / 64][group][row % 64] of this expert
            S.sbr[m] = make_rsrc((const uint32_t*)q.scales + rows0 * G, (uint32_t)N * G * 4);
            continue;
        }
        const rsrc_t rs_s = make_rsrc(q.scales + rows0 * G, (uint32_t)N * G * 2);
        const rsrc_t rs_b = make_rsrc(q.biases + rows0 * G, (uint32_t)N * G * 2);
        const int pieces = ROWS * G / 8;
        uint16_t* dsc = sSc + m * ROWS * GS;
        uint16_t* dbi = sBi + m * ROWS * GS;
        for (int pc = tid; pc < pieces; pc += NT) {
            const int voff = (n_base * G + pc * 8) * 2;
            const u32x4_t vs = __builtin_bit_cast(u32x4_t, __builtin_amdgcn_raw_buffer_load_b128(rs_s, voff, 0, 0));
            const u32x4_t vb = __builtin_bit_cast(u32x4_t, __builtin_amdgcn_raw_buffer_load_b128(rs_b, voff, 0, 0));
            if ((G & 7) == 0) {   // a piece is 8 groups of one row
                const int row = (pc * 8) / G, grp = (pc * 8) % G;
                *(u32x4_t*)(dsc + row * GS + grp) = vs;
                *(u32x4_t*)(dbi + row * GS + grp) = vb;
            } else {
#pragma unroll
                for (int e = 0; e < 8; ++e) {
                    const int flat = pc * 8 + e;
                    const int row = flat / G, grp = flat % G;
                    dsc[row * GS + grp] = (uint16_t)(vs[e / 2] >> (16 * (e & 1)));
                    dbi[row * GS + grp] = (uint16_t)(vb[e / 2] >> (16 * (e & 1)));
                }
            }
        }
    }
    const int row_lane = wave * NSUB * 16 + nl;     // lane's row within the tile
    S.tiles = false;
    if constexpr (BF) {
        S.voff_c = (n_base + row_lane) * (K * 2) + g * W * 16;
        S.sub_c = 16 * (K * 2);
    } else {
        S.tiles = (is_sh ? p.sB[0] : p.rB[0]).layout != 0;
        S.voff_c = (n_base + row_lane) * (K / 2) + g * W * 4;
        S.sub_c = 16 * (K / 2);
        S.chunk_c = KC / 2;
        if (S.tiles) {
            // 64-row tiles x 64-K blocks of 2 KB (16-row groups of 512 B, rows of 32 B);
            // this wave's first 16-row group is rg0 of the workgroup's tile-aligned rows
            const int rg0 = wave * NSUB;
            const int kb = g * W * 8;                    // lane's first weight in the chunk
            auto group_off = [&](int rg) { return (rg / 4) * (K / 64) * 2048 + (rg % 4) * 512; };
            S.voff_c = (n_base / 64) * (K / 64) * 2048 + group_off(rg0) + (kb / 64) * 2048 +
                       nl * 32 + (kb % 64) / 2;
#pragma unroll
            for (int s = 0; s < NSUB; ++s) S.sub_off[s] = group_off(rg0 + s) - group_off(rg0);
            S.chunk_c = (KC / 64) * 2048;
        }
    }
    const int lane_grp = (g * (KC / 4)) / 64;
    if constexpr (SB) {
#pragma unroll
        for (int s = 0; s < NSUB; ++s) {
            const int r = n_base + row_lane + 16 * s;   // row within the expert's matrix
            S.sb_off[s] = (((r / 64) * G + lane_grp) * 64 + r % 64) * 4;
        }
        S.sb_chunk = (KC / 64) * 64 * 4;
    }
    const uint16_t* sSc_lane = sSc + row_lane * GS + lane_grp;
    const uint16_t* sBi_lane = sBi + row_lane * GS + lane_grp;
    const int mstride = ROWS * GS;
    const float unit_inv = 1.0f / fp8_unit();
    const int msub_act = (nr + 15) / 16;

    f32x4_t acc[NMAT][NSUB][MSUB];
#pragma unroll
    for (int m = 0; m < NMAT; ++m)
#pragma unroll
        for (int s = 0; s < NSUB; ++s)
#pragma unroll
            for (int i = 0; i < MSUB; ++i) acc[m][s][i] = f32x4_t{0.f, 0.f, 0.f, 0.f};

    __syncthreads();   // s_row
    const rsrc_t a_rs = make_rsrc(A, (uint32_t)a_rows * lda * 2);
    int a_voff[APT], a_lds[APT];
    bool a_ok[APT];
#pragma unroll
    for (int i = 0; i < APT; ++i) {
        const int q = tid + NT * i;
        a_ok[i] = q < A_PIECES;
        const int qq = a_ok[i] ? q : 0;
        const int row = qq / (KC / 8), c8 = qq % (KC / 8);
        a_voff[i] = s_row[row] * lda * 2 + c8 * 16;
        a_lds[i] = row * LDA + c8 * 8;
    }
    constexpr bool kAllA = A_PIECES % NT == 0;   // every thread holds APT pieces
    auto load_a = [&](u32x4_t (&dst)[APT], int c, int voff_oob) {
#pragma unroll
        for (int i = 0; i < APT; ++i)
            if (kAllA || a_ok[i])
                dst[i] = __builtin_bit_cast(
                    u32x4_t, __builtin_amdgcn_raw_buffer_load_b128(a_rs, a_voff[i] + voff_oob,
                                                                    c * KC * 2, 0));
    };
    auto store_a = [&](const u32x4_t (&src)[APT], uint16_t* dst) {
#pragma unroll
        for (int i = 0; i < APT; ++i)
            if (kAllA || a_ok[i]) *(u32x4_t*)(dst + a_lds[i]) = src[i];
    };

    const int nchunks = K / KC;
    if constexpr (XL) {
        // Direct-to-LDS x rows: the tile of a chunk is MT rows x KC bf16, dense,
        // written as 1 KB blocks (64 lanes x 16 B: RPB rows), block b by wave
        // b % WAVES; lane l of a block writes piece position l % PPR of row
        // b * RPB + l / PPR and fetches the row's piece (l % PPR) ^ (row % 16)
        // (the XOR swizzle that keeps the MFMA fragment reads conflict-free).
        // Chunk c goes to sX[c % 3], requested two chunks ahead, after the
        // chunk's code words; every pipeline step issues NVM vector loads, so
        // waiting for at most NVM outstanding at the end of step c means the
        // x rows of chunk c + 1 (requested in step c - 1) have landed in every
        // wave's part of the tile once the barrier is passed.
        constexpr int PPR = KC / 8, RPB = 64 / PPR, NBLK = MT / RPB;
        static_assert(NBLK % WAVES == 0, "whole 1 KB blocks per wave");
        constexpr int APW = NBLK / WAVES;
        constexpr int NB = NMAT * NSUB * 2;       // code-word and packed-word loads per chunk
        constexpr int NVM = NB + APW;
        int x_voff[APW];
#pragma unroll
        for (int i = 0; i < APW; ++i) {
            const int row = (i * WAVES + wave) * RPB + lane / PPR;
            x_voff[i] = s_row[row] * lda * 2 + (((lane % PPR) ^ (row % 16)) * 16);
        }
        auto load_x = [&](uint16_t* buf, int c, int voff_oob) {
#pragma unroll
            for (int i = 0; i < APW; ++i)
                buffer_load_lds16(a_rs, buf + (i * WAVES + wave) * 512, x_voff[i] + voff_oob,
                                  c * KC * 2);
        };
        auto xbuf = [&](int i) { return i == 0 ? sX0 : (i == 1 ? sX1 : sX2); };
        // The loop is instantiated for both cache policies of the weight words and
        // the item picks one (a branch per load would cost more than the hint
        // gains): non-temporal when this row block is its expert's only one, so
        // the tile is read once and streams through without evicting the x rows
        // and the data the rest of the call reuses; the default when other blocks
        // of the expert read the same tiles from the caches.
        auto xl_loop = [&](auto policy) {
        constexpr bool ST = decltype(policy)::value;
        BChunk<NMAT, NSUB, W, BF> Bq[2];
        load_b<NMAT, NSUB, KC, BF, SB, ST>(Bq[0], S, 0, 0);
        load_x(sX0, 0, 0);
        load_x(sX1, 1, nchunks > 1 ? 0 : kVoffOob);
        MOE_WAIT_VM(APW);
        bare_barrier();
        for (int c0 = 0; c0 < nchunks; c0 += 6) {
#pragma unroll
            for (int d = 0; d < 6; ++d) {
                const int c = c0 + d;
                load_b<NMAT, NSUB, KC, BF, SB, ST>(Bq[(d + 1) % 2], S, c + 1,
                                                   c + 1 < nchunks ? 0 : kVoffOob);
                load_x(xbuf((d + 2) % 3), c + 2, c + 2 < nchunks ? 0 : kVoffOob);
                if (c < nchunks)
                    compute_chunk<NMAT, MT, KC, NSUB, BF, SB, true>(
                        Bq[d % 2], xbuf(d % 3), sSc_lane, sBi_lane, GS, mstride, c * KC / 64,
                        unit_inv, nl, g, msub_act, acc);
                MOE_WAIT_VM(NVM);
                bare_barrier();
            }
        }
        MOE_WAIT_VM(0);   // run-out loads write zeros into the ring: all land before sX0 is reused
        bare_barrier();
        };
        const bool read_once =
            is_sh ? p.sh_blocks == 1 : p.offsets[expert + 1] - p.offsets[expert] <= MT;
        if (read_once) xl_loop(BoolTag<true>{});
        else xl_loop(BoolTag<false>{});
    } else {
        // Register pipeline over K-chunks: the A rows and code words of chunk c
        // live in Aq/Bq[c % DEPTH] and are requested DEPTH-1 chunks before the
        // chunk's math, so no load latency sits between two barriers.  A chunk c
        // is staged into LDS buffer c % 2 one chunk ahead of its math.  Requests
        // past the last chunk go out of bounds (kVoffOob) and are never used.
        BChunk<NMAT, NSUB, W, BF> Bq[DEPTH];
        u32x4_t Aq[DEPTH][APT];
    #pragma unroll
        for (int d = 0; d < DEPTH - 1; ++d) {
            const int oob = d < nchunks ? 0 : kVoffOob;
            load_a(Aq[d], d, oob);
            load_b<NMAT, NSUB, KC, BF, SB>(Bq[d], S, d, oob);
        }
        store_a(Aq[0], sA);
        __syncthreads();
        for (int c0 = 0; c0 < nchunks; c0 += DEPTH) {
    #pragma unroll
            for (int d = 0; d < DEPTH; ++d) {
                const int c = c0 + d;
                const int cp = c + DEPTH - 1;
                const int oob = cp < nchunks ? 0 : kVoffOob;
                load_a(Aq[(d + DEPTH - 1) % DEPTH], cp, oob);
                load_b<NMAT, NSUB, KC, BF, SB>(Bq[(d + DEPTH - 1) % DEPTH], S, cp, oob);
                if (c < nchunks) {
                    compute_chunk<NMAT, MT, KC, NSUB, BF, SB>(Bq[d], sA + (c & 1) * MT * LDA, sSc_lane,
                                                      sBi_lane, GS, mstride, c * KC / 64, unit_inv, nl,
                                                      g, msub_act, acc);
                    // after the last chunk this stages unused data into the idle buffer
                    store_a(Aq[(d + 1) % DEPTH], sA + ((c + 1) & 1) * MT * LDA);
                }
                __syncthreads();
            }
        }

    }

    // ---- epilogue: bf16 tile [MT][COLS] in LDS, then 16-byte row stores ----
    uint16_t* sO = XL ? sX0 : smem_g;
#pragma unroll
    for (int s = 0; s < NSUB; ++s) {
        const int col = (wave * NSUB + s) * 16 + nl;
#pragma unroll
        for (int mi = 0; mi < MSUB; ++mi)
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const int row = mi * 16 + 4 * g + i;
                float v;
                if constexpr (NMAT == 2) v = silu_f32(acc[0][s][mi][i]) * acc[1][s][mi][i];
                else v = acc[0][s][mi][i];
                sO[row * COLS + col] = __builtin_bit_cast(uint16_t, (__bf16)v);
            }
    }
    __syncthreads();
    constexpr int PIECES = MT * COLS / 8;
    const int ncols = min(COLS, N - n_base);
    for (int q = tid; q < PIECES; q += NT) {
        const int row = q / (COLS / 8), c8 = (q % (COLS / 8)) * 8;
        if (row < nr && c8 < ncols)
            *(u32x4_t*)(out + (size_t)(r0 + row) * N + n_base + c8) =
                *(const u32x4_t*)(sO + row * COLS + c8);
    }
}

// ---- Down projection over whole-K tiles (K = I <= 512) ----
// Work item = one row block (MT = 32 rows, or 64 from two blocks, below) x
// CG = WAVES * TPW * 32 output columns.  The block's h rows (MT x K bf16) are
// staged in LDS once per item and every wave reads them; each wave owns TPW
// tiles of 32 output columns over the whole K and requests all of their code
// words right after the h rows, then its lanes' scales and biases, so the item
// streams its weights in one round of loads (the math waits for that round:
// a wave's words arrive as one burst, and requesting the scales first so that
// tile 0 could start earlier measured no faster).  A lane's scales and biases
// for a tile are K / 128 consecutive groups of its weight row, loaded straight
// into registers (8 bytes per array at K = 512): the item keeps no scale table
// in LDS, which lets one more workgroup share a CU.  The product is
// v_mfma_f32_32x32x16_bf16: lane half hf (lane / 32) takes the words of the
// second half of K when hf = 1, so each lane reads half a weight row (K / 4
// bytes) contiguously and its A elements come from the same K positions.
// The dequantization and its arithmetic are those of grouped_q4_kernel
// (dequant_word), so both kernels produce the same weights.
// MT = 64 pairs the row blocks of the 32-row map: block 2i of an expert (counted
// from its first block) takes its own rows and those of block 2i+1, which
// exits at once; the shared expert is cut into 64-row slots (sh_blocks set for
// 64 rows by the host).
template <int KW, int TPW, int WAVES, int MT = 32>
__global__ __launch_bounds__(WAVES * 64) void down_tiles_kernel(GroupedArgs p, int br) {
    constexpr int K = KW * 64;            // weights per row (the down K = I)
    constexpr int NT = WAVES * 64;
    constexpr int LDH = K + 8;            // h row stride in LDS, elements
    constexpr int G = KW;                 // scale groups per weight row
    constexpr int CG = WAVES * TPW * 32;  // output columns per item
    constexpr int CGS = CG + 8;           // output tile row stride in LDS
    constexpr int WPL = 4 * KW;           // code words per lane per tile (half a row)
    constexpr int NGL = KW >= 2 ? KW / 2 : 1;   // scale groups per lane per tile
    constexpr int MR = MT / 32;           // 32-row MFMA tiles per item
    static_assert(WAVES % 2 == 0, "tile-packed offsets assume 64-row steps per tile round");
    extern __shared__ __attribute__((aligned(16))) uint16_t smem_d[];
    uint16_t* sH = smem_d;                // [MT][LDH]
    uint16_t* sO = smem_d;                // [MT][CGS], after the math (aliases sH)

    const int tid = threadIdx.x;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6), lane = tid & 63;
    const int n = lane & 31, hf = lane >> 5;

    const int n_items = (p.sh_blocks + p.n_blocks[0]) * p.n_tiles;
    const int per = (n_items + kXcds - 1) / kXcds;
    const int xcd = blockIdx.x % kXcds, seq = blockIdx.x / kXcds;
    const int item = xcd * per + seq;
    if (seq >= per || item >= n_items) return;
    const int slot = item / p.n_tiles, grp = item % p.n_tiles;
    const bool is_sh = slot < p.sh_blocks;
    int r0, nr, expert = 0;
    if (is_sh) {
        r0 = slot * MT;
        nr = min(MT, p.T - r0);
    } else {
        const int b = slot - p.sh_blocks;
        expert = p.block_expert[b];
        r0 = p.block_row[b];
        if (MT > br && ((r0 - p.offsets[expert]) / br) % (MT / br) != 0) return;   // a follower
        nr = min(MT, p.offsets[expert + 1] - r0);
    }
    const int N = is_sh ? p.N_sh : p.N;
    const int n_base = grp * CG;
    if (n_base >= N) return;   // uniform per workgroup
    const uint16_t* A = is_sh ? p.a_shared : p.a_routed;
    const int lda = is_sh ? p.lda_shared : p.lda_routed;
    const int a_rows = is_sh ? p.rows_shared : p.rows_routed;
    uint16_t* out = is_sh ? p.out_shared : p.out_routed;
    const QMatDev& q = is_sh ? p.sB[0] : p.rB[0];
    const size_t rows0 = (size_t)expert * N;

    // ---- h rows of the block (contiguous; padding rows repeat the last row) ----
    constexpr int HPIECES = MT * (K / 8);
    constexpr int HPT = (HPIECES + NT - 1) / NT;
    const rsrc_t ra = make_rsrc(A, (uint32_t)a_rows * lda * 2);
    u32x4_t hv[HPT];
#pragma unroll
    for (int t = 0; t < HPT; ++t) {
        const int qq = tid + NT * t;
        if (HPIECES % NT == 0 || qq < HPIECES) {
            const int row = qq / (K / 8), c8 = qq % (K / 8);
            hv[t] = __builtin_bit_cast(
                u32x4_t, __builtin_amdgcn_raw_buffer_load_b128(
                             ra, (r0 + min(row, nr - 1)) * lda * 2 + c8 * 16, 0, 0));
        }
    }
    // ---- all code words of the wave's TPW tiles, requested after the h rows so
    // that the h stores below wait only for those ----
    // Tile i of this wave covers output columns n_base + (i*WAVES + wave)*32 ..+32;
    // lane (n, hf) reads words hf*WPL .. +WPL of row (column) n of the tile,
    // KW loads of 4 words.  The per-(tile, load) step is uniform in both word
    // orders and rides in the scalar offset; tiles past N are requested
    // outside the buffer resource (zeros, no memory access).
    const rsrc_t rc = make_rsrc(q.codes + rows0 * (K / 8), (uint32_t)N * (K / 2));
    const int layout = q.layout;
    const int voff = (int)code_word(layout, (uint32_t)(n_base + wave * 32 + n), (uint32_t)(hf * WPL),
                                    (uint32_t)K) * 4;
    u32x4_t Bq[TPW][KW];
#pragma unroll
    for (int i = 0; i < TPW; ++i) {
        const bool ok = n_base + (i * WAVES + wave) * 32 < N;
        const int vo = voff + (ok ? 0 : kVoffOob);
#pragma unroll
        for (int j = 0; j < KW; ++j) {
            const int so = layout == 0
                               ? i * WAVES * 32 * (K / 2) + 16 * j
                               : i * (WAVES / 2) * (K / 64) * 2048 + (KW >= 2 ? (j / 2) * 2048 + (j % 2) * 16 : 0);
            Bq[i][j] = __builtin_bit_cast(u32x4_t, __builtin_amdgcn_raw_buffer_load_b128(rc, vo, so, 0));
        }
    }
    // ---- the lane's NGL groups of its weight row per tile (rows are G bf16 apart in
    // the scale and bias arrays; tiles past N read zeros) ----
    const rsrc_t rs = make_rsrc(q.scales + rows0 * G, (uint32_t)N * G * 2);
    const rsrc_t rb = make_rsrc(q.biases + rows0 * G, (uint32_t)N * G * 2);
    uint32_t lsc[TPW][(NGL + 1) / 2], lbi[TPW][(NGL + 1) / 2];
#pragma unroll
    for (int i = 0; i < TPW; ++i) {
        const int row = n_base + (i * WAVES + wave) * 32 + n;
        const int vo = (row * G + hf * WPL / 8) * 2 + (row < N ? 0 : kVoffOob);
        if constexpr (NGL == 4) {
            const u32x2_t a = __builtin_bit_cast(u32x2_t, __builtin_amdgcn_raw_buffer_load_b64(rs, vo, 0, 0));
            const u32x2_t b = __builtin_bit_cast(u32x2_t, __builtin_amdgcn_raw_buffer_load_b64(rb, vo, 0, 0));
            lsc[i][0] = a[0];
            lsc[i][1] = a[1];
            lbi[i][0] = b[0];
            lbi[i][1] = b[1];
        } else if constexpr (NGL == 2) {
            lsc[i][0] = __builtin_amdgcn_raw_buffer_load_b32(rs, vo, 0, 0);
            lbi[i][0] = __builtin_amdgcn_raw_buffer_load_b32(rb, vo, 0, 0);
        } else {
            lsc[i][0] = __builtin_amdgcn_raw_buffer_load_b16(rs, vo, 0, 0);
            lbi[i][0] = __builtin_amdgcn_raw_buffer_load_b16(rb, vo, 0, 0);
        }
    }
#pragma unroll
    for (int t = 0; t < HPT; ++t) {
        const int qq = tid + NT * t;
        if (HPIECES % NT == 0 || qq < HPIECES) {
            const int row = qq / (K / 8), c8 = qq % (K / 8);
            *(u32x4_t*)(sH + row * LDH + c8 * 8) = hv[t];
        }
    }
    __syncthreads();

    // ---- math: per tile, WPL words per lane, one MFMA per word ----
    const float unit_inv = 1.0f / fp8_unit();
    const int c0 = hf * WPL;              // lane's first word in the row
    const int mr_act = (nr + 31) / 32;    // 32-row tiles holding rows of this item
    f32x16_t acc[TPW][MR];
#pragma unroll
    for (int i = 0; i < TPW; ++i) {
#pragma unroll
        for (int r = 0; r < MR; ++r)
#pragma unroll
            for (int e = 0; e < 16; ++e) acc[i][r][e] = 0.f;
        if (n_base + (i * WAVES + wave) * 32 >= N) continue;   // uniform per wave
        float sc[NGL], bi[NGL];
#pragma unroll
        for (int gg = 0; gg < NGL; ++gg) {
            sc[gg] = bf16_to_f32((uint16_t)(lsc[i][gg / 2] >> (16 * (gg & 1)))) * unit_inv;
            bi[gg] = bf16_to_f32((uint16_t)(lbi[i][gg / 2] >> (16 * (gg & 1))));
        }
#pragma unroll
        for (int j = 0; j < KW; ++j)
#pragma unroll
            for (int w = 0; w < 4; ++w) {
                const int gl = KW >= 2 ? j / 2 : 0;
                const bf16x8_t bw = dequant_word(Bq[i][j][w], sc[gl], bi[gl]);
#pragma unroll
                for (int r = 0; r < MR; ++r) {
                    if (r > 0 && r >= mr_act) break;   // 32-row tiles past the item's rows
                    const bf16x8_t a =
                        *(const bf16x8_t*)(sH + (r * 32 + n) * LDH + (c0 + 4 * j + w) * 8);
                    acc[i][r] = mfma_32x32x16(a, bw, acc[i][r]);
                }
            }
    }

    // ---- epilogue: bf16 tile [32][CG] in LDS (over sH), then 16-byte row stores ----
    __syncthreads();
#pragma unroll
    for (int i = 0; i < TPW; ++i) {
        const int col = (i * WAVES + wave) * 32 + n;
#pragma unroll
        for (int r = 0; r < MR; ++r)
#pragma unroll
            for (int e = 0; e < 16; ++e) {
                const int row = r * 32 + 8 * (e / 4) + 4 * hf + (e % 4);
                sO[row * CGS + col] = __builtin_bit_cast(uint16_t, (__bf16)acc[i][r][e]);
            }
    }
    __syncthreads();
    constexpr int OPIECES = MT * CG / 8;
    const int ncols = min(CG, N - n_base);
    for (int qq = tid; qq < OPIECES; qq += NT) {
        const int row = qq / (CG / 8), c8 = (qq % (CG / 8)) * 8;
        if (row < nr && c8 < ncols)
            *(u32x4_t*)(out + (size_t)(r0 + row) * N + n_base + c8) =
                *(const u32x4_t*)(sO + row * CGS + c8);
    }
}

template <int KW, int TPW, int WAVES, int MT = 32>
static size_t down_tiles_lds_bytes() {
    constexpr int K = KW * 64, CG = WAVES * TPW * 32;
    const size_t a = (size_t)MT * (K + 8) * 2;
    const size_t o = (size_t)MT * (CG + 8) * 2;
    return a > o ? a : o;
}

// Dynamic LDS bytes of one grouped_q4_kernel instance for K-groups G (with
// packed scale|bias words, SB, there is no scale table, and with 128-K chunks
// the A tiles live in the kernel's static LDS ring: nothing dynamic).
template <int NMAT, int MT, int KC, int NSUB, int WAVES, bool SB = false>
static size_t grouped_lds_bytes(int G, int wg_per_cu) {
    constexpr int LDA = KC + 8;
    constexpr int ROWS = WAVES * NSUB * 16;
    if (SB && KC == 128) return 0;   // x rows in the kernel's static LDS ring
    const size_t a = (size_t)2 * MT * LDA * 2 + (SB ? 0 : (size_t)2 * NMAT * ROWS * (G + 8) * 2);
    const size_t o = (size_t)MT * ROWS * 2;
    size_t bytes = a > o ? a : o;
    if (wg_per_cu > 0) {
        const size_t cap = (size_t)160 * 1024 / (wg_per_cu + 1) + 1024;   // > 1/(n+1) of the CU's LDS
        if (bytes < cap) bytes = cap;
    }
    return bytes;
}

size_t gemm_ws_layout(int T, int I, int I_sh, int k, size_t* off_h, size_t* off_hsh) {
    size_t o = 0;
    *off_h = o;
    o += align_up((size_t)T * k * I * sizeof(uint16_t), 256);
    *off_hsh = o;
    o += align_up((size_t)T * I_sh * sizeof(uint16_t), 256);
    return o;
}

static int pick_kc(int K, int K2, int kc_max) {
    for (int kc = kc_max; kc >= 64; kc >>= 1)
        if (K % kc == 0 && (K2 == 0 || K2 % kc == 0)) return kc;
    return 0;
}

template <int NMAT, int MT, int NSUB, int DEPTH, int WAVES, bool BF, bool SB>
static void launch_mt(const GroupedArgs& a, int kc, int grid, int G, int wg_per_cu,
                      hipStream_t stream) {
#define MOE_LAUNCH(KCV)                                                                          \
    grouped_q4_kernel<NMAT, MT, KCV, NSUB, DEPTH, WAVES, BF, SB><<<                              \
        grid, WAVES * 64, grouped_lds_bytes<NMAT, MT, KCV, NSUB, WAVES, SB>(G, wg_per_cu),        \
        stream>>>(a)
    if (kc == 256) MOE_LAUNCH(256);
    else if (kc == 128) MOE_LAUNCH(128);
    else MOE_LAUNCH(64);
#undef MOE_LAUNCH
}

template <int NMAT, int NSUB, int DEPTH, int WAVES, bool BF = false, bool SB = false>
static void launch_grouped(GroupedArgs a, int mt, int kc, int n_max, int slots, int G,
                           int wg_per_cu, hipStream_t stream) {
    constexpr int cols = WAVES * NSUB * 16;
    a.n_tiles = (n_max + cols - 1) / cols;
    const long long items = (long long)slots * a.n_tiles;
    const int grid = (int)((items + kXcds - 1) / kXcds) * kXcds;
    if (mt == 16) launch_mt<NMAT, 16, NSUB, DEPTH, WAVES, BF, SB>(a, kc, grid, G, wg_per_cu, stream);
    else if (mt == 32) launch_mt<NMAT, 32, NSUB, DEPTH, WAVES, BF, SB>(a, kc, grid, G, wg_per_cu, stream);
    else launch_mt<NMAT, 64, NSUB, DEPTH, WAVES, BF, SB>(a, kc, grid, G, wg_per_cu, stream);
}

static GroupedArgs common_args(const GemmProblem& p) {
    GroupedArgs a{};
    a.k = p.k;
    a.T = p.T;
    a.sorted_assign = p.r.sorted_assign;
    a.block_expert = p.r.block_expert;
    a.block_row = p.r.block_row;
    a.n_blocks = p.r.n_blocks;
    a.offsets = p.r.offsets;
    a.sh_blocks = p.I_sh ? (p.T + p.block_rows - 1) / p.block_rows : 0;
    return a;
}

// gate + up with SwiGLU: A = x (gathered by token), N = I, K = H -> h in ws
static GroupedArgs gateup_args(const GemmProblem& p, void* ws) {
    size_t off_h, off_hsh;
    gemm_ws_layout(p.T, p.I, p.I_sh, p.k, &off_h, &off_hsh);
    GroupedArgs a = common_args(p);
    a.a_routed = p.x;
    a.a_shared = p.x;
    a.lda_routed = a.lda_shared = p.H;
    a.rows_routed = a.rows_shared = p.T;
    a.gather = 1;
    a.rB[0] = p.gate;
    a.rB[1] = p.up;
    a.sB[0] = p.sh_gate;
    a.sB[1] = p.sh_up;
    a.N = p.I;
    a.K = p.H;
    a.N_sh = p.I_sh;
    a.K_sh = p.H;
    a.out_routed = (uint16_t*)((char*)ws + off_h);
    a.out_shared = (uint16_t*)((char*)ws + off_hsh);
    return a;
}

// down: A = h rows (contiguous, from ws), N = H, K = I -> expert_out / shared_out
static GroupedArgs down_args(const GemmProblem& p, const void* ws) {
    size_t off_h, off_hsh;
    gemm_ws_layout(p.T, p.I, p.I_sh, p.k, &off_h, &off_hsh);
    GroupedArgs a = common_args(p);
    a.a_routed = (const uint16_t*)((const char*)ws + off_h);
    a.a_shared = (const uint16_t*)((const char*)ws + off_hsh);
    a.lda_routed = p.I;
    a.lda_shared = p.I_sh;
    a.rows_routed = p.T * p.k;
    a.rows_shared = p.T;
    a.gather = 0;
    a.rB[0] = p.down;
    a.sB[0] = p.sh_down;
    a.N = p.H;
    a.K = p.I;
    a.N_sh = p.I_sh ? p.H : 0;
    a.K_sh = p.I_sh;
    a.out_routed = p.expert_out;
    a.out_shared = p.shared_out;
    return a;
}

hipError_t launch_gateup(const GemmProblem& p, void* ws, hipStream_t stream) {
    const GroupedArgs a = gateup_args(p, ws);
    if (p.gate.layout == 2) {   // packed scale|bias words: no LDS table, a shorter ring
        launch_grouped<2, MOE_GU_NSUB, MOE_GU_SB_DEPTH, MOE_GU_WAVES, false, true>(
            a, p.block_rows, pick_kc(p.H, 0, MOE_GU_KC), p.I > p.I_sh ? p.I : p.I_sh,
            a.sh_blocks + p.max_blocks, p.H / 64, MOE_GU_WG_PER_CU, stream);
        return hipGetLastError();
    }
    launch_grouped<2, MOE_GU_NSUB, MOE_GU_DEPTH, MOE_GU_WAVES>(
        a, p.block_rows, pick_kc(p.H, 0, MOE_GU_KC), p.I > p.I_sh ? p.I : p.I_sh,
        a.sh_blocks + p.max_blocks, p.H / 64, MOE_GU_WG_PER_CU, stream);
    return hipGetLastError();
}

#ifndef MOE_DT_WAVES
#define MOE_DT_WAVES 4
#endif
#ifndef MOE_DT_TPW
#define MOE_DT_TPW 2
#endif

#ifndef MOE_DP_WAVES
#define MOE_DP_WAVES 8
#endif
#ifndef MOE_DP_TPW
#define MOE_DP_TPW 1
#endif

template <int KW, int TPW, int WAVES, int MT>
static void launch_down_tiles_mt(GroupedArgs a, int br, int n_max, int slots, hipStream_t stream) {
    constexpr int cg = WAVES * TPW * 32;
    a.n_tiles = (n_max + cg - 1) / cg;
    const long long items = (long long)slots * a.n_tiles;
    const int grid = (int)((items + kXcds - 1) / kXcds) * kXcds;
    down_tiles_kernel<KW, TPW, WAVES, MT>
        <<<grid, WAVES * 64, down_tiles_lds_bytes<KW, TPW, WAVES, MT>(), stream>>>(a, br);
}

// 64-row items (pairs of 32-row blocks) when the experts average at least
// MOE_DP_MIN_ROWS rows: each dequantized weight then feeds up to 64 rows.
#ifndef MOE_DP_MIN_ROWS
#define MOE_DP_MIN_ROWS 48
#endif

template <int KW>
static void launch_down_tiles(GroupedArgs a, const GemmProblem& p, hipStream_t stream) {
    const bool pair = p.block_rows == 32 && (long long)p.T * p.k >= (long long)MOE_DP_MIN_ROWS * p.E;
    if (pair) {
        a.sh_blocks = p.I_sh ? (p.T + 63) / 64 : 0;
        launch_down_tiles_mt<KW, MOE_DP_TPW, MOE_DP_WAVES, 64>(a, p.block_rows, p.H,
                                                              a.sh_blocks + p.max_blocks, stream);
    } else {
        launch_down_tiles_mt<KW, MOE_DT_TPW, MOE_DT_WAVES, 32>(a, p.block_rows, p.H,
                                                              a.sh_blocks + p.max_blocks, stream);
    }
}

// The whole-K tile kernel serves row blocks of up to 32 rows with one K
// (routed and shared) of 64, 128, 256 or 512; other shapes take the
// K-chunked grouped kernel.
static bool down_tiles_fits(const GemmProblem& p) {
#ifdef MOE_DT_DISABLE
    return false;
#endif
    if (p.block_rows > 32) return false;
    if (p.I_sh && p.I_sh != p.I) return false;
    return p.I == 64 || p.I == 128 || p.I == 256 || p.I == 512;
}

hipError_t launch_down(const GemmProblem& p, const void* ws, hipStream_t stream) {
    const GroupedArgs a = down_args(p, ws);
    if (down_tiles_fits(p)) {
        if (p.I == 512) launch_down_tiles<8>(a, p, stream);
        else if (p.I == 256) launch_down_tiles<4>(a, p, stream);
        else if (p.I == 128) launch_down_tiles<2>(a, p, stream);
        else launch_down_tiles<1>(a, p, stream);
        return hipGetLastError();
    }
    launch_grouped<1, MOE_DN_NSUB, MOE_DN_DEPTH, MOE_DN_WAVES>(
        a, p.block_rows, pick_kc(p.I, p.I_sh, MOE_DN_KC), p.H, a.sh_blocks + p.max_blocks,
        (p.I > p.I_sh ? p.I : p.I_sh) / 64, MOE_DN_WG_PER_CU, stream);
    return hipGetLastError();
}

// The same two phases over weights already expanded to bf16 in memory (the
// unfused baseline).  A bf16 chunk is 4x the bytes of a 4-bit one, so the
// K-chunk is halved to keep the register ring the same size.
constexpr int kBfKc = 64;

hipError_t launch_gateup_bf16(const GemmProblem& p, const uint16_t* const w[4], void* ws,
                              hipStream_t stream) {
    GroupedArgs a = gateup_args(p, ws);
    a.rW[0] = w[0];
    a.rW[1] = w[1];
    a.sW[0] = w[2];
    a.sW[1] = w[3];
    launch_grouped<2, MOE_GU_NSUB, MOE_GU_DEPTH, MOE_GU_WAVES, true>(
        a, p.block_rows, pick_kc(p.H, 0, kBfKc), p.I > p.I_sh ? p.I : p.I_sh,
        a.sh_blocks + p.max_blocks, p.H / 64, MOE_GU_WG_PER_CU, stream);
    return hipGetLastError();
}

hipError_t launch_down_bf16(const GemmProblem& p, const uint16_t* down, const uint16_t* sh_down,
                            const void* ws, hipStream_t stream) {
    GroupedArgs a = down_args(p, ws);
    a.rW[0] = down;
    a.sW[0] = sh_down;
    launch_grouped<1, MOE_DN_NSUB, MOE_DN_DEPTH, MOE_DN_WAVES, true>(
        a, p.block_rows, pick_kc(p.I, p.I_sh, kBfKc), p.H, a.sh_blocks + p.max_blocks,
        (p.I > p.I_sh ? p.I : p.I_sh) / 64, MOE_DN_WG_PER_CU, stream);
    return hipGetLastError();
}

}  // namespace moeq4
