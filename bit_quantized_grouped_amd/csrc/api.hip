// C ABI of the 4-bit grouped MoE layer: host-side validation, workspace
// layout and kernel dispatch.  Every entry point checks all of its arguments
// before its first launch and enqueues nothing when a check fails; none
// allocates, frees or synchronises.  A multi-kernel call can still return
// MOE_ERR_HIP from a later launch after its earlier kernels were enqueued.
#include <initializer_list>
#include <mutex>
#include <new>

#include "../../include/moe_q4.h"
#include "moe_launch.h"

using namespace moeq4;

namespace {

constexpr int kAbiVersion = 5;
constexpr int kMaxE = 1000;

bool aligned(const void* p, size_t a) { return ((uintptr_t)p % a) == 0; }

bool valid_block_rows(int br) { return br == 16 || br == 32 || br == 64; }

int check_route_shape(int T, int E, int k, int block_rows) {
    if (T < 1 || E < 1 || E > kMaxE || k < 1 || k > E) return MOE_ERR_SHAPE;
    if (!valid_block_rows(block_rows)) return MOE_ERR_SHAPE;
    if ((long long)T * k >= (1ll << 30)) return MOE_ERR_SHAPE;
    return MOE_OK;
}

int check_layer_shape(int T, int H, int I, int I_sh, int E, int k, int block_rows) {
    const int st = check_route_shape(T, E, k, block_rows);
    if (st) return st;
    if (H < 64 || H % 64 || I < 64 || I % 64 || I_sh < 0 || I_sh % 64) return MOE_ERR_SHAPE;
    // the kernels form 32-bit byte offsets inside one buffer: bf16 rows of x, h,
    // expert_out and shared_out, and one expert's code words
    const long long widest = H > I ? H : I;
    if ((long long)T * k * widest >= (1ll << 30)) return MOE_ERR_SHAPE;
    if ((long long)T * (I_sh > H ? I_sh : H) >= (1ll << 30)) return MOE_ERR_SHAPE;
    if ((long long)H * (I > I_sh ? I : I_sh) >= (1ll << 32)) return MOE_ERR_SHAPE;
    return MOE_OK;
}

int check_mat(const moe_q4_mat* m) {
    if (!m || !m->codes || !m->scales) return MOE_ERR_NULL;
    if (m->layout == MOE_Q4_LAYOUT_TILES_SB) {   // packed scale|bias words; biases not read
        if (!aligned(m->codes, 16) || !aligned(m->scales, 4)) return MOE_ERR_ALIGN;
        return MOE_OK;
    }
    if (!m->biases) return MOE_ERR_NULL;
    if (!aligned(m->codes, 16) || !aligned(m->scales, 2) || !aligned(m->biases, 2))
        return MOE_ERR_ALIGN;
    if (m->layout != MOE_Q4_LAYOUT_ROWS && m->layout != MOE_Q4_LAYOUT_TILES) return MOE_ERR_SHAPE;
    return MOE_OK;
}

// Every non-NULL matrix of one call shares the first one's layout.
static int check_same_layout(std::initializer_list<const moe_q4_mat*> mats) {
    int layout = -1;
    for (const moe_q4_mat* m : mats) {
        if (!m) continue;
        if (layout < 0) layout = m->layout;
        else if (m->layout != layout) return MOE_ERR_SHAPE;
    }
    return MOE_OK;
}

static int code_order(const moe_q4_mat* m) {
    return m->layout == MOE_Q4_LAYOUT_ROWS ? MOE_Q4_LAYOUT_ROWS : MOE_Q4_LAYOUT_TILES;
}

// The layout rules of one layer's matrices (NULL ones skipped): gate, up, sh_gate and sh_up
// share one layout; down and sh_down share one, which is not TILES_SB; all share one
// code-word order.
static int check_layer_layouts(const moe_q4_mat* gate, const moe_q4_mat* up,
                               const moe_q4_mat* down, const moe_q4_mat* sh_gate,
                               const moe_q4_mat* sh_up, const moe_q4_mat* sh_down) {
    int st = check_same_layout({gate, up, sh_gate, sh_up});
    if (st || (st = check_same_layout({down, sh_down}))) return st;
    int order = -1;
    for (const moe_q4_mat* m : {gate, up, down, sh_gate, sh_up, sh_down}) {
        if (!m) continue;
        if (order < 0) order = code_order(m);
        else if (code_order(m) != order) return MOE_ERR_SHAPE;
    }
    for (const moe_q4_mat* m : {down, sh_down})
        if (m && m->layout == MOE_Q4_LAYOUT_TILES_SB) return MOE_ERR_SHAPE;
    return MOE_OK;
}

int check_routing(const moe_routing* r) {
    if (!r || !r->topk_idx || !r->topk_w || !r->counts || !r->offsets || !r->sorted_assign ||
        !r->assign_row || !r->block_expert || !r->block_row || !r->n_blocks)
        return MOE_ERR_NULL;
    return MOE_OK;
}

int max_blocks_of(int T, int E, int k, int br) {
    const long long n = (long long)T * k;
    return (int)((n + br - 1) / br + (E < n ? E : n));
}

RoutingDev to_dev(const moe_routing* r) {
    return RoutingDev{r->topk_idx, r->topk_w,        r->counts,       r->offsets,  r->sorted_assign,
                      r->assign_row, r->block_expert, r->block_row, r->n_blocks};
}

QMatDev to_dev(const moe_q4_mat* m) {
    if (!m) return QMatDev{nullptr, nullptr, nullptr, 0};
    return QMatDev{m->codes, m->scales, m->biases, m->layout};
}

// Layout of moe_layer_chunked's workspace for chunks of C tokens.
struct LayerWs {
    size_t topk_idx, topk_w, counts, offsets, sorted_assign, assign_row, block_expert, block_row,
        n_blocks, route_ws, gemm_ws, expert_out, shared_out, total;
    size_t route_bytes, gemm_bytes;
};

LayerWs layer_ws_layout(int C, int H, int I, int I_sh, int E, int k, int br) {
    LayerWs L{};
    const size_t n = (size_t)C * k;
    const size_t mb = (size_t)max_blocks_of(C, E, k, br);
    size_t o = 0;
    auto take = [&](size_t bytes) {
        const size_t at = o;
        o += align_up(bytes, 256);
        return at;
    };
    L.topk_idx = take(n * 4);
    L.topk_w = take(n * 4);
    L.counts = take((size_t)E * 4);
    L.offsets = take((size_t)(E + 1) * 4);
    L.sorted_assign = take(n * 4);
    L.assign_row = take(n * 4);
    L.block_expert = take(mb * 4);
    L.block_row = take(mb * 4);
    L.n_blocks = take(4);
    size_t a, b;
    L.route_bytes = route_ws_layout(C, E, k, &a, &b);
    L.route_ws = take(L.route_bytes);
    L.gemm_bytes = gemm_ws_layout(C, I, I_sh, k, &a, &b);
    L.gemm_ws = take(L.gemm_bytes);
    L.expert_out = take(n * H * 2);
    L.shared_out = take(I_sh ? (size_t)C * H * 2 : 0);
    L.total = o;
    return L;
}

int gemm_args_ok(const uint16_t* x, int T, int H, int I, int I_sh, int E, int k, int block_rows,
                 const moe_routing* r, const moe_q4_mat* gate, const moe_q4_mat* up,
                 const moe_q4_mat* down, const moe_q4_mat* sh_gate, const moe_q4_mat* sh_up,
                 const moe_q4_mat* sh_down, const uint16_t* expert_out,
                 const uint16_t* shared_out) {
    int st = check_layer_shape(T, H, I, I_sh, E, k, block_rows);
    if (st) return st;
    if (!x || !expert_out) return MOE_ERR_NULL;
    if ((st = check_routing(r))) return st;
    if ((st = check_mat(gate)) || (st = check_mat(up)) || (st = check_mat(down))) return st;
    if (I_sh) {
        if (!shared_out) return MOE_ERR_NULL;
        if ((st = check_mat(sh_gate)) || (st = check_mat(sh_up)) || (st = check_mat(sh_down)))
            return st;
        if (!aligned(shared_out, 16)) return MOE_ERR_ALIGN;
    } else if (sh_gate || sh_up || sh_down || shared_out) {
        return MOE_ERR_SHAPE;   // shared matrices given but I_sh == 0
    }
    if ((st = check_layer_layouts(gate, up, down, sh_gate, sh_up, sh_down))) return st;
    if (!aligned(x, 16) || !aligned(expert_out, 16)) return MOE_ERR_ALIGN;
    return MOE_OK;
}

}  // namespace

extern "C" {

int moe_abi_version(void) { return kAbiVersion; }

const char* moe_status_str(int status) {
    switch (status) {
        case MOE_OK: return "ok";
        case MOE_ERR_NULL: return "null pointer";
        case MOE_ERR_SHAPE: return "bad shape";
        case MOE_ERR_ALIGN: return "misaligned pointer";
        case MOE_ERR_WORKSPACE: return "workspace too small";
        case MOE_ERR_HIP: return "HIP launch error";
        case MOE_ERR_UNIMPLEMENTED: return "unimplemented";
        default: return "unknown status";
    }
}

int moe_route_max_blocks(int T, int E, int k, int block_rows) {
    const int st = check_route_shape(T, E, k, block_rows);
    if (st) return st;
    return max_blocks_of(T, E, k, block_rows);
}

size_t moe_route_workspace_bytes(int T, int E, int k, int block_rows) {
    if (check_route_shape(T, E, k, block_rows)) return 0;
    size_t a, b;
    return route_ws_layout(T, E, k, &a, &b);
}

int moe_route(const float* logits, int T, int E, int k, int block_rows, const moe_routing* out,
              void* ws, size_t ws_bytes, hipStream_t stream) {
    try {
        int st = check_route_shape(T, E, k, block_rows);
        if (st) return st;
        const size_t need = moe_route_workspace_bytes(T, E, k, block_rows);
        if (!logits || (need && !ws)) return MOE_ERR_NULL;
        if ((st = check_routing(out))) return st;
        if (!aligned(logits, 4) || !aligned(ws, 256)) return MOE_ERR_ALIGN;
        if (ws_bytes < need) return MOE_ERR_WORKSPACE;
        const hipError_t e = launch_route(logits, T, E, k, block_rows,
                                          max_blocks_of(T, E, k, block_rows), to_dev(out), ws,
                                          stream);
        return e == hipSuccess ? MOE_OK : MOE_ERR_HIP;
    } catch (...) {
        return MOE_ERR_HIP;
    }
}

size_t moe_gemm_workspace_bytes(int T, int H, int I, int I_sh, int E, int k, int block_rows) {
    if (check_layer_shape(T, H, I, I_sh, E, k, block_rows)) return 0;
    size_t a, b;
    return gemm_ws_layout(T, I, I_sh, k, &a, &b);
}

static GemmProblem make_problem(const uint16_t* x, int T, int H, int I, int I_sh, int E, int k,
                                int block_rows, const moe_routing* r, const moe_q4_mat* gate,
                                const moe_q4_mat* up, const moe_q4_mat* down,
                                const moe_q4_mat* sh_gate, const moe_q4_mat* sh_up,
                                const moe_q4_mat* sh_down, uint16_t* expert_out,
                                uint16_t* shared_out) {
    GemmProblem p{};
    p.x = x;
    p.T = T;
    p.H = H;
    p.I = I;
    p.I_sh = I_sh;
    p.E = E;
    p.k = k;
    p.block_rows = block_rows;
    p.max_blocks = max_blocks_of(T, E, k, block_rows);
    p.r = to_dev(r);
    p.gate = to_dev(gate);
    p.up = to_dev(up);
    p.down = to_dev(down);
    p.sh_gate = to_dev(sh_gate);
    p.sh_up = to_dev(sh_up);
    p.sh_down = to_dev(sh_down);
    p.expert_out = expert_out;
    p.shared_out = shared_out;
    return p;
}

static int check_ws(const void* ws, size_t ws_bytes, size_t need) {
    if (!ws) return MOE_ERR_NULL;
    if (!aligned(ws, 256)) return MOE_ERR_ALIGN;
    if (ws_bytes < need) return MOE_ERR_WORKSPACE;
    return MOE_OK;
}

// One validated layer call: route, gate/up, down and combine in stream order.
static int layer_call(const GemmProblem& p, const float* logits, void* route_ws, void* gemm_ws,
                      uint16_t* y, hipStream_t stream) {
    hipError_t e =
        launch_route(logits, p.T, p.E, p.k, p.block_rows, p.max_blocks, p.r, route_ws, stream);
    if (e == hipSuccess) e = launch_gateup(p, gemm_ws, stream);
    if (e == hipSuccess) e = launch_down(p, gemm_ws, stream);
    if (e == hipSuccess)
        e = launch_combine(p.expert_out, p.shared_out, nullptr, p.r.assign_row, p.r.topk_w, p.T,
                           p.H, p.k, y, stream);
    return e == hipSuccess ? MOE_OK : MOE_ERR_HIP;
}

int moe_grouped_gemm_q4(const uint16_t* x, int T, int H, int I, int I_sh, int E, int k,
                        int block_rows, const moe_routing* r, const moe_q4_mat* gate,
                        const moe_q4_mat* up, const moe_q4_mat* down, const moe_q4_mat* sh_gate,
                        const moe_q4_mat* sh_up, const moe_q4_mat* sh_down, uint16_t* expert_out,
                        uint16_t* shared_out, void* ws, size_t ws_bytes, hipStream_t stream) {
    try {
        int st = gemm_args_ok(x, T, H, I, I_sh, E, k, block_rows, r, gate, up, down, sh_gate,
                              sh_up, sh_down, expert_out, shared_out);
        if (st) return st;
        if ((st = check_ws(ws, ws_bytes, moe_gemm_workspace_bytes(T, H, I, I_sh, E, k, block_rows))))
            return st;
        const GemmProblem p = make_problem(x, T, H, I, I_sh, E, k, block_rows, r, gate, up, down,
                                           sh_gate, sh_up, sh_down, expert_out, shared_out);
        hipError_t e = launch_gateup(p, ws, stream);
        if (e == hipSuccess) e = launch_down(p, ws, stream);
        return e == hipSuccess ? MOE_OK : MOE_ERR_HIP;
    } catch (...) {
        return MOE_ERR_HIP;
    }
}

int moe_layer_q4(const uint16_t* x, const float* logits, int T, int H, int I, int I_sh, int E,
                 int k, int block_rows, const moe_q4_mat* gate, const moe_q4_mat* up,
                 const moe_q4_mat* down, const moe_q4_mat* sh_gate, const moe_q4_mat* sh_up,
                 const moe_q4_mat* sh_down, const moe_routing* r, void* route_ws,
                 size_t route_ws_bytes, uint16_t* expert_out, uint16_t* shared_out,
                 void* gemm_ws, size_t gemm_ws_bytes, uint16_t* y, hipStream_t stream) {
    try {
        int st = gemm_args_ok(x, T, H, I, I_sh, E, k, block_rows, r, gate, up, down, sh_gate,
                              sh_up, sh_down, expert_out, shared_out);
        if (st) return st;
        if (!logits || !y) return MOE_ERR_NULL;
        if (!aligned(logits, 4) || !aligned(y, 16)) return MOE_ERR_ALIGN;
        const size_t route_need = moe_route_workspace_bytes(T, E, k, block_rows);
        if (route_need && (st = check_ws(route_ws, route_ws_bytes, route_need))) return st;
        if ((st = check_ws(gemm_ws, gemm_ws_bytes,
                           moe_gemm_workspace_bytes(T, H, I, I_sh, E, k, block_rows))))
            return st;
        const GemmProblem p = make_problem(x, T, H, I, I_sh, E, k, block_rows, r, gate, up, down,
                                           sh_gate, sh_up, sh_down, expert_out, shared_out);
        return layer_call(p, logits, route_ws, gemm_ws, y, stream);
    } catch (...) {
        return MOE_ERR_HIP;
    }
}

int moe_expert_gateup_q4(const uint16_t* x, int T, int H, int I, int I_sh, int E, int k,
                         int block_rows, const moe_routing* r, const moe_q4_mat* gate,
                         const moe_q4_mat* up, const moe_q4_mat* sh_gate,
                         const moe_q4_mat* sh_up, void* ws, size_t ws_bytes,
                         hipStream_t stream) {
    try {
        int st = check_layer_shape(T, H, I, I_sh, E, k, block_rows);
        if (st) return st;
        if (!x) return MOE_ERR_NULL;
        if ((st = check_routing(r))) return st;
        if ((st = check_mat(gate)) || (st = check_mat(up))) return st;
        if (I_sh) {
            if ((st = check_mat(sh_gate)) || (st = check_mat(sh_up))) return st;
        } else if (sh_gate || sh_up) {
            return MOE_ERR_SHAPE;
        }
        if ((st = check_same_layout({gate, up, sh_gate, sh_up}))) return st;
        if (!aligned(x, 16)) return MOE_ERR_ALIGN;
        if ((st = check_ws(ws, ws_bytes, moe_gemm_workspace_bytes(T, H, I, I_sh, E, k, block_rows))))
            return st;
        const GemmProblem p = make_problem(x, T, H, I, I_sh, E, k, block_rows, r, gate, up,
                                           nullptr, sh_gate, sh_up, nullptr, nullptr, nullptr);
        return launch_gateup(p, ws, stream) == hipSuccess ? MOE_OK : MOE_ERR_HIP;
    } catch (...) {
        return MOE_ERR_HIP;
    }
}

int moe_expert_down_q4(int T, int H, int I, int I_sh, int E, int k, int block_rows,
                       const moe_routing* r, const moe_q4_mat* down, const moe_q4_mat* sh_down,
                       uint16_t* expert_out, uint16_t* shared_out, const void* ws,
                       size_t ws_bytes, hipStream_t stream) {
    try {
        int st = check_layer_shape(T, H, I, I_sh, E, k, block_rows);
        if (st) return st;
        if (!expert_out) return MOE_ERR_NULL;
        if ((st = check_routing(r))) return st;
        if ((st = check_mat(down))) return st;
        if ((st = check_layer_layouts(nullptr, nullptr, down, nullptr, nullptr, sh_down))) return st;
        if (I_sh) {
            if (!shared_out) return MOE_ERR_NULL;
            if ((st = check_mat(sh_down))) return st;
            if (!aligned(shared_out, 16)) return MOE_ERR_ALIGN;
        } else if (sh_down || shared_out) {
            return MOE_ERR_SHAPE;
        }
        if (!aligned(expert_out, 16)) return MOE_ERR_ALIGN;
        if ((st = check_ws(ws, ws_bytes, moe_gemm_workspace_bytes(T, H, I, I_sh, E, k, block_rows))))
            return st;
        const GemmProblem p = make_problem(nullptr, T, H, I, I_sh, E, k, block_rows, r, nullptr,
                                           nullptr, down, nullptr, nullptr, sh_down, expert_out,
                                           shared_out);
        return launch_down(p, ws, stream) == hipSuccess ? MOE_OK : MOE_ERR_HIP;
    } catch (...) {
        return MOE_ERR_HIP;
    }
}

int moe_q4_prepack(const uint32_t* src_codes, int n_exp, int N, int K, uint32_t* dst_codes,
                   hipStream_t stream) {
    try {
        if (n_exp < 1 || N < 64 || N % 64 || K < 64 || K % 64) return MOE_ERR_SHAPE;
        if ((size_t)n_exp * N * (K / 8) >= ((size_t)1 << 31)) return MOE_ERR_SHAPE;
        if (!src_codes || !dst_codes) return MOE_ERR_NULL;
        if (src_codes == dst_codes) return MOE_ERR_SHAPE;
        if (!aligned(src_codes, 16) || !aligned(dst_codes, 16)) return MOE_ERR_ALIGN;
        return launch_prepack(src_codes, n_exp, N, K, dst_codes, stream) == hipSuccess
                   ? MOE_OK
                   : MOE_ERR_HIP;
    } catch (...) {
        return MOE_ERR_HIP;
    }
}

int moe_q4_pack_scales(const uint16_t* scales, const uint16_t* biases, int n_exp, int N, int K,
                       uint32_t* dst, hipStream_t stream) {
    try {
        if (n_exp < 1 || N < 64 || N % 64 || K < 64 || K % 64) return MOE_ERR_SHAPE;
        if ((size_t)n_exp * N * (K / 64) >= ((size_t)1 << 31)) return MOE_ERR_SHAPE;
        if (!scales || !biases || !dst) return MOE_ERR_NULL;
        if ((const void*)dst == (const void*)scales || (const void*)dst == (const void*)biases)
            return MOE_ERR_SHAPE;
        if (!aligned(scales, 2) || !aligned(biases, 2) || !aligned(dst, 4)) return MOE_ERR_ALIGN;
        return launch_pack_scales(scales, biases, n_exp, N, K, dst, stream) == hipSuccess
                   ? MOE_OK
                   : MOE_ERR_HIP;
    } catch (...) {
        return MOE_ERR_HIP;
    }
}

int moe_dequant_q4_bf16(const moe_q4_mat* m, int n_exp, int N, int K, const int32_t* counts,
                        uint16_t* out, hipStream_t stream) {
    try {
        if (n_exp < 1 || N < 1 || K < 64 || K % 64) return MOE_ERR_SHAPE;
        if ((size_t)n_exp * N * (K / 8) >= ((size_t)1 << 31)) return MOE_ERR_SHAPE;
        int st = check_mat(m);
        if (st) return st;
        if (m->layout != MOE_Q4_LAYOUT_ROWS) return MOE_ERR_UNIMPLEMENTED;   // expands row-major codes
        if (!out) return MOE_ERR_NULL;
        if (!aligned(out, 16)) return MOE_ERR_ALIGN;
        return launch_dequant_bf16(to_dev(m), n_exp, N, K, counts, out, stream) == hipSuccess
                   ? MOE_OK
                   : MOE_ERR_HIP;
    } catch (...) {
        return MOE_ERR_HIP;
    }
}

static int check_bf16_weights(const uint16_t* w) {
    if (!w) return MOE_ERR_NULL;
    return aligned(w, 16) ? MOE_OK : MOE_ERR_ALIGN;
}

int moe_expert_gateup_bf16(const uint16_t* x, int T, int H, int I, int I_sh, int E, int k,
                           int block_rows, const moe_routing* r, const uint16_t* gate,
                           const uint16_t* up, const uint16_t* sh_gate, const uint16_t* sh_up,
                           void* ws, size_t ws_bytes, hipStream_t stream) {
    try {
        int st = check_layer_shape(T, H, I, I_sh, E, k, block_rows);
        if (st) return st;
        // one expert's bf16 matrix (4x its code bytes) also stays below 2^31 bytes
        if ((long long)H * (I > I_sh ? I : I_sh) >= (1ll << 30)) return MOE_ERR_SHAPE;
        if (!x) return MOE_ERR_NULL;
        if ((st = check_routing(r))) return st;
        if ((st = check_bf16_weights(gate)) || (st = check_bf16_weights(up))) return st;
        if (I_sh) {
            if ((st = check_bf16_weights(sh_gate)) || (st = check_bf16_weights(sh_up))) return st;
        } else if (sh_gate || sh_up) {
            return MOE_ERR_SHAPE;
        }
        if (!aligned(x, 16)) return MOE_ERR_ALIGN;
        if ((st = check_ws(ws, ws_bytes, moe_gemm_workspace_bytes(T, H, I, I_sh, E, k, block_rows))))
            return st;
        const GemmProblem p = make_problem(x, T, H, I, I_sh, E, k, block_rows, r, nullptr, nullptr,
                                           nullptr, nullptr, nullptr, nullptr, nullptr, nullptr);
        const uint16_t* const w[4] = {gate, up, sh_gate, sh_up};
        return launch_gateup_bf16(p, w, ws, stream) == hipSuccess ? MOE_OK : MOE_ERR_HIP;
    } catch (...) {
        return MOE_ERR_HIP;
    }
}

int moe_expert_down_bf16(int T, int H, int I, int I_sh, int E, int k, int block_rows,
                         const moe_routing* r, const uint16_t* down, const uint16_t* sh_down,
                         uint16_t* expert_out, uint16_t* shared_out, const void* ws,
                         size_t ws_bytes, hipStream_t stream) {
    try {
        int st = check_layer_shape(T, H, I, I_sh, E, k, block_rows);
        if (st) return st;
        // one expert's bf16 matrix (4x its code bytes) also stays below 2^31 bytes
        if ((long long)H * (I > I_sh ? I : I_sh) >= (1ll << 30)) return MOE_ERR_SHAPE;
        if (!expert_out) return MOE_ERR_NULL;
        if ((st = check_routing(r))) return st;
        if ((st = check_bf16_weights(down))) return st;
        if (I_sh) {
            if (!shared_out) return MOE_ERR_NULL;
            if ((st = check_bf16_weights(sh_down))) return st;
            if (!aligned(shared_out, 16)) return MOE_ERR_ALIGN;
        } else if (sh_down || shared_out) {
            return MOE_ERR_SHAPE;
        }
        if (!aligned(expert_out, 16)) return MOE_ERR_ALIGN;
        if ((st = check_ws(ws, ws_bytes, moe_gemm_workspace_bytes(T, H, I, I_sh, E, k, block_rows))))
            return st;
        const GemmProblem p = make_problem(nullptr, T, H, I, I_sh, E, k, block_rows, r, nullptr,
                                           nullptr, nullptr, nullptr, nullptr, nullptr, expert_out,
                                           shared_out);
        return launch_down_bf16(p, down, sh_down, ws, stream) == hipSuccess ? MOE_OK : MOE_ERR_HIP;
    } catch (...) {
        return MOE_ERR_HIP;
    }
}

int moe_combine(const uint16_t* expert_out, const uint16_t* shared_out, const moe_routing* r,
                int T, int H, int k, uint16_t* y, hipStream_t stream) {
    try {
        if (T < 1 || k < 1 || H < 64 || H % 64) return MOE_ERR_SHAPE;
        if ((long long)T * k * H >= (1ll << 30)) return MOE_ERR_SHAPE;
        if (!expert_out || !y || !r || !r->assign_row || !r->topk_w) return MOE_ERR_NULL;
        if (!aligned(expert_out, 16) || !aligned(y, 16) || (shared_out && !aligned(shared_out, 16)))
            return MOE_ERR_ALIGN;
        const hipError_t e =
            launch_combine(expert_out, shared_out, nullptr, r->assign_row, r->topk_w, T, H, k, y, stream);
        return e == hipSuccess ? MOE_OK : MOE_ERR_HIP;
    } catch (...) {
        return MOE_ERR_HIP;
    }
}

int moe_combine_gated(const uint16_t* expert_out, const uint16_t* shared_out,
                      const float* shared_gate, const moe_routing* r, int T, int H, int k,
                      uint16_t* y, hipStream_t stream) {
    try {
        if (T < 1 || k < 1 || H < 64 || H % 64) return MOE_ERR_SHAPE;
        if ((long long)T * k * H >= (1ll << 30)) return MOE_ERR_SHAPE;
        if (!expert_out || !shared_out || !shared_gate || !y || !r || !r->assign_row || !r->topk_w)
            return MOE_ERR_NULL;
        if (!aligned(expert_out, 16) || !aligned(y, 16) || !aligned(shared_out, 16) ||
            !aligned(shared_gate, 4))
            return MOE_ERR_ALIGN;
        const hipError_t e = launch_combine(expert_out, shared_out, shared_gate, r->assign_row,
                                            r->topk_w, T, H, k, y, stream);
        return e == hipSuccess ? MOE_OK : MOE_ERR_HIP;
    } catch (...) {
        return MOE_ERR_HIP;
    }
}

int moe_router(const uint16_t* x, int T, int H, const uint16_t* w_router, int E,
               const uint16_t* w_gate, float* logits, float* gate, hipStream_t stream) {
    try {
        if (T < 1 || H < 64 || H % 64 || E < 1 || E > 1000) return MOE_ERR_SHAPE;
        if (!x || !w_router || !logits) return MOE_ERR_NULL;
        if ((w_gate == nullptr) != (gate == nullptr)) return MOE_ERR_NULL;
        if (!aligned(x, 16) || !aligned(w_router, 16) || !aligned(logits, 4) ||
            (w_gate && !aligned(w_gate, 16)) || (gate && !aligned(gate, 4)))
            return MOE_ERR_ALIGN;
        return launch_router(x, T, H, w_router, E, w_gate, logits, gate, stream) == hipSuccess
                   ? MOE_OK
                   : MOE_ERR_HIP;
    } catch (...) {
        return MOE_ERR_HIP;
    }
}

size_t moe_read_probe_sink_words(size_t bytes) { return read_probe_sink_words(bytes); }

int moe_read_probe(const void* buf, size_t bytes, uint32_t* sink, size_t sink_words,
                   hipStream_t stream) {
    try {
        if (!buf || !sink) return MOE_ERR_NULL;
        if (bytes < 16 || bytes % 16 || bytes / 16 > ((size_t)1 << 40)) return MOE_ERR_SHAPE;
        if (!aligned(buf, 16) || !aligned(sink, 4)) return MOE_ERR_ALIGN;
        if (sink_words < read_probe_sink_words(bytes)) return MOE_ERR_WORKSPACE;
        if (read_probe_sink_words(bytes) > 0x7fffffffu) return MOE_ERR_SHAPE;
        return launch_read_probe(buf, bytes, sink, stream) == hipSuccess ? MOE_OK : MOE_ERR_HIP;
    } catch (...) {
        return MOE_ERR_HIP;
    }
}

int moe_launch_probe(uint32_t* buf, int n_launches, int grid_a, int threads_a, int grid_b,
                     int threads_b, int dep, hipStream_t stream) {
    try {
        if (!buf) return MOE_ERR_NULL;
        if (!aligned(buf, 4)) return MOE_ERR_ALIGN;
        auto bad_shape = [](int g, int t) { return g < 1 || g > 65535 || t < 64 || t > 1024 || t % 64; };
        if (n_launches < 1 || bad_shape(grid_a, threads_a) || bad_shape(grid_b, threads_b) ||
            (dep != 0 && dep != 1))
            return MOE_ERR_SHAPE;
        return launch_launch_probe(buf, n_launches, grid_a, threads_a, grid_b, threads_b, dep,
                                   stream) == hipSuccess
                   ? MOE_OK
                   : MOE_ERR_HIP;
    } catch (...) {
        return MOE_ERR_HIP;
    }
}

size_t moe_decode_workspace_bytes(int H, int I, int I_sh, int E, int k) {
    if (check_layer_shape(1, H, I, I_sh, E, k, 32) || k > 64) return 0;
    return decode_ws_layout(H, I, I_sh, k).total;
}

}  // extern "C"

namespace {

// Host-side checks of one decode call (everything but the workspace); fills
// the kernel arguments except the workspace pointers.
int decode_args(const uint16_t* x, const float* logits, int H, int I, int I_sh, int E, int k,
                int block_rows, const moe_q4_mat* gate, const moe_q4_mat* up,
                const moe_q4_mat* down, const moe_q4_mat* sh_gate, const moe_q4_mat* sh_up,
                const moe_q4_mat* sh_down, const moe_routing* r, uint16_t* y, DecodeArgs* a) {
    int st = check_layer_shape(1, H, I, I_sh, E, k, block_rows);
    if (st) return st;
    if (k > 64) return MOE_ERR_SHAPE;
    if (!x || !logits || !y) return MOE_ERR_NULL;
    if ((st = check_mat(gate)) || (st = check_mat(up)) || (st = check_mat(down))) return st;
    if (I_sh) {
        if ((st = check_mat(sh_gate)) || (st = check_mat(sh_up)) || (st = check_mat(sh_down)))
            return st;
    } else if (sh_gate || sh_up || sh_down) {
        return MOE_ERR_SHAPE;
    }
    if ((st = check_layer_layouts(gate, up, down, sh_gate, sh_up, sh_down))) return st;
    if (r && (st = check_routing(r))) return st;
    if (!aligned(x, 16) || !aligned(y, 16) || !aligned(logits, 4)) return MOE_ERR_ALIGN;
    *a = DecodeArgs{};
    a->x = x;
    a->logits = logits;
    a->H = H;
    a->I = I;
    a->I_sh = I_sh;
    a->E = E;
    a->k = k;
    a->gate = to_dev(gate);
    a->up = to_dev(up);
    a->down = to_dev(down);
    a->sh_gate = to_dev(sh_gate);
    a->sh_up = to_dev(sh_up);
    a->sh_down = to_dev(sh_down);
    a->write_routing = r ? 1 : 0;
    if (r) a->r = to_dev(r);
    a->max_blocks = max_blocks_of(1, E, k, block_rows);
    a->y = y;
    return MOE_OK;
}

// Points the decode kernels' workspace (h, then the chosen experts and their
// weights) at ws.
void decode_ws(DecodeArgs* a, void* ws) {
    const DecodeWs L = decode_ws_layout(a->H, a->I, a->I_sh, a->k);
    a->h = (uint16_t*)((char*)ws + L.h);
    a->sel_idx = (int32_t*)((char*)ws + L.sel_idx);
    a->sel_w = (float*)((char*)ws + L.sel_w);
}

// ---- scratch for moe_decode_q4_noalloc ----
// A file-scope device array stands in for the workspace of callers that cannot
// allocate.  In host code `decode_scratch` names a host-side stand-in, not a
// device address: its device address is looked up once per device with
// hipGetSymbolAddress (that device current) and only that address is used.
constexpr size_t kDecodeScratchBytes = 256 * 1024;
constexpr int kMaxDevices = 64;
__device__ __align__(256) unsigned char decode_scratch[kDecodeScratchBytes];
std::mutex g_scratch_mu;
void* g_scratch_ptr[kMaxDevices] = {};

// Device address of decode_scratch on the device that owns `stream`.
hipError_t scratch_for(hipStream_t stream, void** out) {
    int dev = 0;
    hipError_t e = stream ? hipStreamGetDevice(stream, &dev) : hipGetDevice(&dev);
    if (e != hipSuccess) return e;
    if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
    std::lock_guard<std::mutex> lock(g_scratch_mu);
    if (!g_scratch_ptr[dev]) {
        int cur = 0;
        if ((e = hipGetDevice(&cur)) != hipSuccess) return e;
        if (cur != dev && (e = hipSetDevice(dev)) != hipSuccess) return e;
        void* p = nullptr;
        e = hipGetSymbolAddress(&p, HIP_SYMBOL(decode_scratch));
        if (cur != dev) {
            const hipError_t e2 = hipSetDevice(cur);
            if (e == hipSuccess) e = e2;
        }
        if (e != hipSuccess) return e;
        if (!p) return hipErrorInvalidSymbol;
        g_scratch_ptr[dev] = p;
    }
    *out = g_scratch_ptr[dev];
    return hipSuccess;
}

}  // namespace

extern "C" {

int moe_decode_q4(const uint16_t* x, const float* logits, int H, int I, int I_sh, int E, int k,
                  int block_rows, const moe_q4_mat* gate, const moe_q4_mat* up,
                  const moe_q4_mat* down, const moe_q4_mat* sh_gate, const moe_q4_mat* sh_up,
                  const moe_q4_mat* sh_down, const moe_routing* r, uint16_t* y, void* ws,
                  size_t ws_bytes, hipStream_t stream) {
    try {
        DecodeArgs a;
        int st = decode_args(x, logits, H, I, I_sh, E, k, block_rows, gate, up, down, sh_gate,
                             sh_up, sh_down, r, y, &a);
        if (st) return st;
        if ((st = check_ws(ws, ws_bytes, decode_ws_layout(H, I, I_sh, k).total))) return st;
        decode_ws(&a, ws);
        return launch_decode(a, stream) == hipSuccess ? MOE_OK : MOE_ERR_HIP;
    } catch (...) {
        return MOE_ERR_HIP;
    }
}

size_t moe_decode_noalloc_max_bytes(void) { return kDecodeScratchBytes; }

int moe_decode_q4_noalloc(const uint16_t* x, const float* logits, int H, int I, int I_sh, int E,
                          int k, int block_rows, const moe_q4_mat* gate, const moe_q4_mat* up,
                          const moe_q4_mat* down, const moe_q4_mat* sh_gate,
                          const moe_q4_mat* sh_up, const moe_q4_mat* sh_down,
                          const moe_routing* r, uint16_t* y, hipStream_t stream) {
    try {
        DecodeArgs a;
        int st = decode_args(x, logits, H, I, I_sh, E, k, block_rows, gate, up, down, sh_gate,
                             sh_up, sh_down, r, y, &a);
        if (st) return st;
        if (decode_ws_layout(H, I, I_sh, k).total > kDecodeScratchBytes)
            return MOE_ERR_WORKSPACE;
        void* scratch = nullptr;
        if (scratch_for(stream, &scratch) != hipSuccess) return MOE_ERR_HIP;
        decode_ws(&a, scratch);
        return launch_decode(a, stream) == hipSuccess ? MOE_OK : MOE_ERR_HIP;
    } catch (...) {
        return MOE_ERR_HIP;
    }
}

int moe_decode_q4_sequential(const uint16_t* x, const float* logits, int n_tok, int H, int I,
                             int I_sh, int E, int k, const moe_q4_mat* gate,
                             const moe_q4_mat* up, const moe_q4_mat* down,
                             const moe_q4_mat* sh_gate, const moe_q4_mat* sh_up,
                             const moe_q4_mat* sh_down, uint16_t* y, void* ws, size_t ws_bytes,
                             hipStream_t stream) {
    if (n_tok < 1) return MOE_ERR_SHAPE;
    // validate once through the single-token entry's checks (token 0 pointers)
    for (int t = 0; t < n_tok; ++t) {
        const int st = moe_decode_q4(x + (size_t)t * H, logits + (size_t)t * E, H, I, I_sh, E, k,
                                     32, gate, up, down, sh_gate, sh_up, sh_down, nullptr,
                                     y + (size_t)t * H, ws, ws_bytes, stream);
        if (st) return st;
    }
    return MOE_OK;
}

size_t moe_layer_workspace_bytes(int chunk_tokens, int H, int I, int I_sh, int E, int k,
                                 int block_rows) {
    if (check_layer_shape(chunk_tokens, H, I, I_sh, E, k, block_rows)) return 0;
    return layer_ws_layout(chunk_tokens, H, I, I_sh, E, k, block_rows).total;
}

int moe_layer_chunked(const uint16_t* x, const float* logits, int T, int H, int I, int I_sh,
                      int E, int k, int block_rows, int chunk_tokens, const moe_q4_mat* gate,
                      const moe_q4_mat* up, const moe_q4_mat* down, const moe_q4_mat* sh_gate,
                      const moe_q4_mat* sh_up, const moe_q4_mat* sh_down, uint16_t* y, void* ws,
                      size_t ws_bytes, hipStream_t stream) {
    try {
        if (chunk_tokens < 1) return MOE_ERR_SHAPE;
        const int C = chunk_tokens < T ? chunk_tokens : T;
        // Every kernel works inside one chunk (x, logits and y are advanced on the
        // host in size_t), so the 31-bit offset limits apply to the chunk; the whole
        // prompt only needs a valid routing shape.
        int st = check_route_shape(T, E, k, block_rows);
        if (st) return st;
        if ((st = check_layer_shape(C, H, I, I_sh, E, k, block_rows))) return st;
        if (!x || !logits || !y || !ws) return MOE_ERR_NULL;
        if ((st = check_mat(gate)) || (st = check_mat(up)) || (st = check_mat(down))) return st;
        if (I_sh) {
            if ((st = check_mat(sh_gate)) || (st = check_mat(sh_up)) || (st = check_mat(sh_down)))
                return st;
        } else if (sh_gate || sh_up || sh_down) {
            return MOE_ERR_SHAPE;
        }
        if ((st = check_layer_layouts(gate, up, down, sh_gate, sh_up, sh_down))) return st;
        if (!aligned(x, 16) || !aligned(y, 16) || !aligned(logits, 4) || !aligned(ws, 256))
            return MOE_ERR_ALIGN;
        const LayerWs L = layer_ws_layout(C, H, I, I_sh, E, k, block_rows);
        if (ws_bytes < L.total) return MOE_ERR_WORKSPACE;
        char* base = (char*)ws;
        moe_routing r{};
        r.topk_idx = (int32_t*)(base + L.topk_idx);
        r.topk_w = (float*)(base + L.topk_w);
        r.counts = (int32_t*)(base + L.counts);
        r.offsets = (int32_t*)(base + L.offsets);
        r.sorted_assign = (int32_t*)(base + L.sorted_assign);
        r.assign_row = (int32_t*)(base + L.assign_row);
        r.block_expert = (int32_t*)(base + L.block_expert);
        r.block_row = (int32_t*)(base + L.block_row);
        r.n_blocks = (int32_t*)(base + L.n_blocks);
        uint16_t* eo = (uint16_t*)(base + L.expert_out);
        uint16_t* so = I_sh ? (uint16_t*)(base + L.shared_out) : nullptr;
        for (int t0 = 0; t0 < T; t0 += C) {
            const int Tc = (T - t0) < C ? (T - t0) : C;
            const GemmProblem p = make_problem(x + (size_t)t0 * H, Tc, H, I, I_sh, E, k,
                                               block_rows, &r, gate, up, down, sh_gate, sh_up,
                                               sh_down, eo, so);
            st = layer_call(p, logits + (size_t)t0 * E, base + L.route_ws, base + L.gemm_ws,
                            y + (size_t)t0 * H, stream);
            if (st) return st;
        }
        return MOE_OK;
    } catch (...) {
        return MOE_ERR_HIP;
    }
}

}  // extern "C"
