// C ABI of libloopvq: argument validation, buffer layout and launch
// configuration.  Everything before the kernel launch is plain host
// arithmetic, so every error path returns before any HIP call.
#include "../../include/loopvq.h"
#include "../../include/loopvq_diag.h"

#include <algorithm>
#include <cmath>
#include <cstdint>
#include <cstring>

#include "kernels.h"

namespace {

// KV heads: the heads of the index caches, codebooks and windows
int64_t kv_heads(const lvq_config *c) { return c->n_kv_heads > 0 ? c->n_kv_heads : c->n_heads; }
// R: loop steps of the model; R / Tc index rows (groups) per token
int64_t n_loops(const lvq_config *c) { return c->n_loops > 0 ? c->n_loops : c->loop_steps; }

bool config_ok(const lvq_config *c) {
    if (!c) return false;
    if (c->batch < 1 || c->n_heads < 1 || c->head_dim < 1) return false;
    if (c->loop_steps < 1 || c->group < 1) return false;
    if (c->group % c->loop_steps != 0) return false;
    const int cg = c->group / c->loop_steps;
    if (c->head_dim % cg != 0) return false;
    if (c->n_sink < 0 || c->n_recent < 1 || c->max_tokens < 0) return false;
    if ((int64_t)c->n_sink + c->n_recent > LVQ_MAX_WINDOW_SLOTS) return false;
    if (c->codebook_dtype != LVQ_F32 && c->codebook_dtype != LVQ_BF16) return false;
    if (c->decode_splits < 0 || c->decode_splits > LVQ_MAX_SPLITS) return false;
    if (c->decode_window_groups < 0 || c->decode_window_groups > LVQ_MAX_WINDOW_GROUPS) return false;
    if (c->decode_window_groups > 0 && c->decode_window_groups >= c->decode_splits) return false;
    if (c->batch > 65535 || c->n_heads > 65535) return false;
    if (c->n_kv_heads < 0 || c->n_kv_heads > c->n_heads) return false;
    if (c->n_kv_heads > 0 && c->n_heads % c->n_kv_heads != 0) return false;
    if (c->n_loops < 0 || c->n_loops > LVQ_MAX_LOOPS || c->n_loops % c->loop_steps != 0) return false;
    if (c->decode_poll_limit < 0) return false;
    if (c->decode_heads_per_group < 0 || c->decode_heads_per_group > 2) return false;
    return true;
}

void set_tensor(lvq_tensor *t, int ndim, const int64_t *shape, uint64_t elem_bytes) {
    t->ndim = ndim;
    for (int i = 0; i < 6; ++i) t->shape[i] = t->stride[i] = 0;
    int64_t s = 1;
    for (int i = ndim - 1; i >= 0; --i) {
        t->shape[i] = shape[i];
        t->stride[i] = s;
        s *= shape[i];
    }
    t->bytes = (uint64_t)s * elem_bytes;
}

int64_t max_vq_tokens(const lvq_config *c, int32_t max_ctx_len, bool exact_windows) {
    const int64_t L = max_ctx_len;
    const int64_t n_s = L < c->n_sink ? L : c->n_sink;
    const int64_t v = exact_windows ? L - c->n_sink - c->n_recent : L - n_s;
    return v > 0 ? v : 0;
}

// Workgroups per (b, h) and where the bf16 window slots go, from a cost model
// of the launch.  One decode workgroup fills a compute unit's LDS, so the grid
// runs in ceil(B*H*n / 256) rounds on MI355X's 256 CUs.  A workgroup costs a
// fixed start-up (codebook staging and first loads under a loaded memory
// system, about kFixedBatches token batches' worth) plus the bytes it reads,
// counted in VQ tokens: its VQ tokens, which it folds in whole batches of
// decode_batch_tokens(S), and its bf16 window rows (a window slot reads
// 2 * 2d bytes against 2S for a VQ token: 2d/S VQ tokens).  Every sequence is
// costed at the longest one's length.  When a grid with two workgroups per
// (b, h) fits the chip, only one-round grids are considered, and w extra
// workgroups per (b, h) split the window slots (they need no codebook tables,
// and the last of them merges the others' partials while they finish); a
// round costs its slowest workgroup.  Splits stay at least 512 tokens long;
// ties go to fewer workgroups.
struct Splits {
    int32_t n;          // workgroups per (b, h)
    int32_t n_win;      // the last n_win of them split the window slots (0: none)
};
constexpr int64_t kTargetGroups = 256;
constexpr int32_t kDefaultPolls = 1 << 22;   // a merger's wait: seconds, far beyond any call
constexpr int64_t kFixedBatches = 6;
constexpr int64_t kMaxWindowGroups = LVQ_MAX_WINDOW_GROUPS;

Splits choose_splits(const lvq_config *c, int64_t max_vq, int64_t n_layers = 1, int nh = 1) {
    if (max_vq <= 0) return {1, 0};
    const int64_t bh = n_layers * c->batch * (c->n_heads / nh);   // workgroup groups
    if (c->decode_splits != 0) {
        int64_t want = c->decode_splits;
        if (want < 1) want = 1;
        if (want > LVQ_MAX_SPLITS) want = LVQ_MAX_SPLITS;
        const int32_t w = c->decode_window_groups > 0 ? c->decode_window_groups : 1;
        return {(int32_t)want, want > 1 && bh * want <= kTargetGroups ? w : 0};
    }
    const int S = c->head_dim / (c->group / c->loop_steps);
    const int64_t step = lvq::decode_batch_tokens(S);
    const int64_t W = (int64_t)c->n_sink + c->n_recent;
    const int64_t wslot = 2 * (int64_t)c->head_dim / S;    // VQ tokens per window slot
    int64_t best_cost = -1, best_n = 1, best_win = 0;
    auto consider = [&](int64_t cost, int64_t n, int64_t n_win) {
        if (best_cost < 0 || cost < best_cost || (cost == best_cost && n < best_n)) {
            best_cost = cost;
            best_n = n;
            best_win = n_win;
        }
    };
    // small grids: one round with window workgroups
    const bool win = bh * 2 <= kTargetGroups;
    for (int64_t n_vq = 1; n_vq < LVQ_MAX_SPLITS; ++n_vq) {
        const int64_t chunk = (max_vq + n_vq - 1) / n_vq;
        if (n_vq > 1 && chunk < 512) break;
        const int64_t vq_cost = ((chunk + step - 1) / step + kFixedBatches) * step;
        if (win) {
            if (bh * (n_vq + 1) > kTargetGroups) break;
            for (int64_t w = 1; w <= kMaxWindowGroups && bh * (n_vq + w) <= kTargetGroups; ++w) {
                const int64_t win_cost = kFixedBatches * step + wslot * ((W + w - 1) / w);
                consider(std::max(vq_cost, win_cost), n_vq + w, w);
            }
        } else {
            const int64_t rounds = (bh * n_vq + kTargetGroups - 1) / kTargetGroups;
            consider(rounds * (vq_cost + wslot * W / n_vq), n_vq, 0);
        }
    }
    return {(int32_t)best_n, best_n > 1 ? (int32_t)best_win : 0};
}

// Query heads per decode workgroup: 2 (two consecutive query heads of one KV
// head read its index rows once) when the kernel has that variant (S = 32,
// cg = 4, bf16 codebooks, head_dim 128, one layer per launch, an even number
// of query heads per KV head) and the plan for head pairs merges through
// window workgroups or needs no merge; otherwise 1.  decode_heads_per_group
// forces 1, or 2 (0 where 2 is not possible).
struct Plan {
    Splits sp;
    int nh;
};
Plan decode_plan(const lvq_config *c, int64_t max_vq, int64_t n_layers) {
    const int want = c->decode_heads_per_group;
    if (want != 1) {
        const int cg = c->group / c->loop_steps;
        const int64_t S = c->head_dim / cg;
        const bool shape = n_layers == 1 && (c->n_heads / kv_heads(c)) % 2 == 0 && S == 32 && cg == 4 &&
                           c->head_dim == 128 && c->codebook_dtype == LVQ_BF16;
        if (shape) {
            const Splits sp = choose_splits(c, max_vq, n_layers, 2);
            if (sp.n == 1 || sp.n_win > 0) return {sp, 2};
        }
        if (want == 2) return {{0, 0}, 0};
    }
    return {choose_splits(c, max_vq, n_layers, 1), 1};
}

// Encode n tensors of one shape (1: lvq_encode; 2: the K and V of a page in one
// launch per group).  Every argument is checked before anything is launched.
lvq_status encode_tensors(const lvq_config *c, int n, const void *const *x, const int64_t *x_strides,
                          int64_t n_tokens, const void *const *codebook, uint8_t *const *index_cache,
                          int32_t seq, int64_t first_token, void *stream, float *screen = nullptr) {
    if (!config_ok(c)) return LVQ_ERR_INVALID_ARG;
    for (int i = 0; i < n; ++i)
        if (!x[i] || !codebook[i] || !index_cache[i]) return LVQ_ERR_INVALID_ARG;
    if (n_tokens < 0 || seq < 0 || seq >= c->batch) return LVQ_ERR_INVALID_ARG;
    if (first_token < 0 || first_token + n_tokens > c->max_tokens) return LVQ_ERR_INVALID_ARG;
    const int cg = c->group / c->loop_steps;
    // the encoder writes the index caches: one pass per KV head, and per group
    // of Tc loop steps when the model has R > Tc
    const int64_t H = kv_heads(c), d = c->head_dim, Tc = c->loop_steps, R = n_loops(c);
    int64_t st[3] = {H * R * d, R * d, d};
    if (x_strides) {
        for (int i = 0; i < 3; ++i) {
            st[i] = x_strides[i];
            if (st[i] < 0 || st[i] % cg != 0) return LVQ_ERR_INVALID_ARG;
        }
    }
    for (int i = 0; i < n; ++i) {
        // sub-vector runs of cg bf16 are read as one vector
        if (reinterpret_cast<uintptr_t>(x[i]) % (2 * (uintptr_t)cg) != 0) return LVQ_ERR_INVALID_ARG;
        // the codebooks are staged in 16-byte pieces
        if (reinterpret_cast<uintptr_t>(codebook[i]) % 16 != 0) return LVQ_ERR_INVALID_ARG;
        // index rows are written a 4-byte word (4 sub-vectors) at a time
        if (reinterpret_cast<uintptr_t>(index_cache[i]) % 4 != 0) return LVQ_ERR_INVALID_ARG;
    }
    // a 32-token tile of one head is addressed with 32-bit byte offsets
    if (2 * (31 * st[0] + Tc * st[2] + d) >= 0x7ffffff0LL) return LVQ_ERR_UNSUPPORTED;
    if (!lvq::encode_supported(c->group, cg, (int)(c->head_dim / cg),
                               c->codebook_dtype == LVQ_BF16))
        return LVQ_ERR_UNSUPPORTED;
    if (n_tokens == 0) return LVQ_OK;
    const size_t cbe = c->codebook_dtype == LVQ_BF16 ? 2 : 4;
    const int64_t S = c->head_dim / cg;
    lvq::EncodeArgs a{};
    a.H = (int)H;
    a.d = c->head_dim;
    a.Tc = c->loop_steps;
    a.G = c->group;
    a.cg = cg;
    a.S = c->head_dim / cg;
    a.cb_bf16 = c->codebook_dtype == LVQ_BF16;
    a.n_tensors = n;
    a.sx_tok = st[0];
    a.sx_head = st[1];
    a.sx_step = st[2];
    a.n_tokens = n_tokens;
    a.t_max = c->max_tokens;
    a.seq = seq;
    a.first_token = first_token;
    a.screen = screen;
    for (int64_t g = 0; g < R / Tc; ++g) {
        // group g: loop steps g*Tc .. g*Tc + Tc - 1, codebook slices of those
        // steps, and the group's index cache block
        const size_t cb_off = (size_t)(g * Tc * H) * LVQ_CODES * S * cg * cbe;
        const size_t idx_off = (size_t)g * c->batch * H * c->max_tokens * S;
        a.x = static_cast<const uint16_t *>(x[0]) + g * Tc * st[2];
        a.cb = static_cast<const char *>(codebook[0]) + cb_off;
        a.index = index_cache[0] + idx_off;
        if (n == 2) {
            a.x_b = static_cast<const uint16_t *>(x[1]) + g * Tc * st[2];
            a.cb_b = static_cast<const char *>(codebook[1]) + cb_off;
            a.index_b = index_cache[1] + idx_off;
        }
        hipError_t e = lvq::launch_encode(a, static_cast<hipStream_t>(stream));
        if (e != hipSuccess) return LVQ_ERR_HIP;
    }
    return LVQ_OK;
}

}  // namespace

extern "C" {

const char *lvq_status_string(lvq_status s) {
    switch (s) {
        case LVQ_OK: return "ok";
        case LVQ_ERR_INVALID_ARG: return "invalid argument";
        case LVQ_ERR_UNSUPPORTED: return "unsupported shape";
        case LVQ_ERR_WORKSPACE: return "workspace missing or too small";
        case LVQ_ERR_HIP: return "HIP launch error";
    }
    return "unknown status";
}

lvq_status lvq_cache_layout(const lvq_config *c, lvq_layout *o) {
    if (!o || !config_ok(c)) return LVQ_ERR_INVALID_ARG;
    std::memset(o, 0, sizeof *o);
    const int64_t B = c->batch, H = c->n_heads, Hk = kv_heads(c), d = c->head_dim, Tc = c->loop_steps;
    const int64_t cg = c->group / c->loop_steps, S = d / cg, W = (int64_t)c->n_sink + c->n_recent;
    const uint64_t cbe = c->codebook_dtype == LVQ_BF16 ? 2 : 4;
    o->n_sub = (int32_t)S;
    o->sub_channels = (int32_t)cg;
    o->n_codes = LVQ_CODES;
    o->window_slots = (int32_t)W;
    o->bits_per_element = 8.0 / (double)c->group;
    o->compression_vs_bf16 = 16.0 / o->bits_per_element;
    // per token and loop step: bf16 K and V read 2 * d * 2 bytes; the index
    // rows (K and V, shared by all loop steps) are re-read whole: 2 * S bytes
    o->read_reduction_per_step = (4.0 * (double)d) / (2.0 * (double)S);
    const int64_t R = n_loops(c), NG = R / Tc;
    if (NG == 1) {
        const int64_t idx_shape[4] = {B, Hk, c->max_tokens, S};
        set_tensor(&o->k_index, 4, idx_shape, 1);
        set_tensor(&o->v_index, 4, idx_shape, 1);
    } else {
        const int64_t idx_shape[5] = {NG, B, Hk, c->max_tokens, S};
        set_tensor(&o->k_index, 5, idx_shape, 1);
        set_tensor(&o->v_index, 5, idx_shape, 1);
    }
    const int64_t cb_shape[5] = {R, Hk, LVQ_CODES, S, cg};
    set_tensor(&o->k_codebook, 5, cb_shape, cbe);
    set_tensor(&o->v_codebook, 5, cb_shape, cbe);
    const int64_t win_shape[5] = {B, R, Hk, W, d};
    set_tensor(&o->k_window, 5, win_shape, 2);
    set_tensor(&o->v_window, 5, win_shape, 2);
    const int64_t q_shape[3] = {B, H, d};
    set_tensor(&o->query, 3, q_shape, 2);
    set_tensor(&o->output, 3, q_shape, 4);
    o->workspace_bytes = lvq::workspace_bytes(B, H);
    return LVQ_OK;
}

int32_t lvq_decode_splits(const lvq_config *c, int32_t max_ctx_len) {
    if (!config_ok(c) || max_ctx_len < 0 || max_ctx_len > c->max_tokens) return 0;
    return decode_plan(c, max_vq_tokens(c, max_ctx_len, true), 1).sp.n;
}

int32_t lvq_decode_window_groups(const lvq_config *c, int32_t max_ctx_len) {
    if (!config_ok(c) || max_ctx_len < 0 || max_ctx_len > c->max_tokens) return -1;
    const Plan plan = decode_plan(c, max_vq_tokens(c, max_ctx_len, true), 1);
    return plan.nh == 0 ? -1 : plan.sp.n_win;
}

int32_t lvq_decode_heads_per_workgroup(const lvq_config *c, int32_t n_layers, int32_t max_ctx_len) {
    if (!config_ok(c) || n_layers < 1 || n_layers > LVQ_MAX_LAYERS) return 0;
    if (max_ctx_len < 0 || max_ctx_len > c->max_tokens) return 0;
    const int64_t nl = n_layers < lvq::kMaxLayersPerLaunch ? n_layers : lvq::kMaxLayersPerLaunch;
    return decode_plan(c, max_vq_tokens(c, max_ctx_len, true), nl).nh;
}

lvq_status lvq_encode(const lvq_config *c, const void *x, const int64_t *x_strides,
                      int64_t n_tokens, const void *codebook, uint8_t *index_cache,
                      int32_t seq, int64_t first_token, void *stream) {
    const void *xs[1] = {x};
    const void *cbs[1] = {codebook};
    uint8_t *idx[1] = {index_cache};
    return encode_tensors(c, 1, xs, x_strides, n_tokens, cbs, idx, seq, first_token, stream);
}

lvq_status lvq_encode_screen(const lvq_config *c, const void *x, const int64_t *x_strides,
                             int64_t n_tokens, const void *codebook, uint8_t *index_cache,
                             int32_t seq, int64_t first_token, float *screen, void *stream) {
    if (!screen) return LVQ_ERR_INVALID_ARG;
    if (config_ok(c) && n_loops(c) != c->loop_steps) return LVQ_ERR_UNSUPPORTED;
    if (reinterpret_cast<uintptr_t>(screen) % 16) return LVQ_ERR_INVALID_ARG;
    const void *xs[1] = {x};
    const void *cbs[1] = {codebook};
    uint8_t *idx[1] = {index_cache};
    return encode_tensors(c, 1, xs, x_strides, n_tokens, cbs, idx, seq, first_token, stream, screen);
}

lvq_status lvq_encode_kv(const lvq_config *c, const void *k_x, const void *v_x,
                         const int64_t *x_strides, int64_t n_tokens, const void *k_codebook,
                         const void *v_codebook, uint8_t *k_index, uint8_t *v_index, int32_t seq,
                         int64_t first_token, void *stream) {
    const void *xs[2] = {k_x, v_x};
    const void *cbs[2] = {k_codebook, v_codebook};
    uint8_t *idx[2] = {k_index, v_index};
    return encode_tensors(c, 2, xs, x_strides, n_tokens, cbs, idx, seq, first_token, stream);
}

namespace {

// Every check of a decode call, then one launch per kMaxLayersPerLaunch
// layers.  Layer l uses the workspace blocks (l * B + b) * H + h after the
// header.
// With use_scratch the workspace is the library's static device array
// (lvq_decode_attn_noalloc): it needs room for the blocks only where a launch
// merges, and its address is looked up once every check has passed.
lvq_status decode_layers(const lvq_config *c, int32_t n_layers, int32_t loop_step,
                         const lvq_decode_layer *layers, const int32_t *ctx_len,
                         const int32_t *vq_len, int32_t max_ctx_len, float sm_scale,
                         void *workspace, uint64_t workspace_bytes, void *stream,
                         bool use_scratch = false) {
    if (!config_ok(c)) return LVQ_ERR_INVALID_ARG;
    if (n_layers < 1 || n_layers > LVQ_MAX_LAYERS || !layers || !ctx_len) return LVQ_ERR_INVALID_ARG;
    if (loop_step < 0 || loop_step >= n_loops(c)) return LVQ_ERR_INVALID_ARG;
    if (max_ctx_len < 0 || max_ctx_len > c->max_tokens) return LVQ_ERR_INVALID_ARG;
    if (c->max_tokens < 1) return LVQ_ERR_INVALID_ARG;     // the index cache has rows
    if (!std::isfinite(sm_scale)) return LVQ_ERR_INVALID_ARG;
    const int cg = c->group / c->loop_steps;
    const int S = c->head_dim / cg;
    for (int32_t l = 0; l < n_layers; ++l) {
        const lvq_decode_layer &L = layers[l];
        if (!L.q || !L.k_index || !L.v_index || !L.k_codebook || !L.v_codebook || !L.k_window ||
            !L.v_window || !L.out)
            return LVQ_ERR_INVALID_ARG;
        // index rows and window rows are read with 8- or 16-byte vector loads
        const uintptr_t ia = S >= 16 ? 16 : 8;
        if (reinterpret_cast<uintptr_t>(L.k_index) % ia || reinterpret_cast<uintptr_t>(L.v_index) % ia)
            return LVQ_ERR_INVALID_ARG;
        if (reinterpret_cast<uintptr_t>(L.k_window) % 16 || reinterpret_cast<uintptr_t>(L.v_window) % 16)
            return LVQ_ERR_INVALID_ARG;
        // the score tables read q in 16-byte pieces
        if (reinterpret_cast<uintptr_t>(L.q) % 16) return LVQ_ERR_INVALID_ARG;
        if (reinterpret_cast<uintptr_t>(L.k_codebook) % 16 ||
            reinterpret_cast<uintptr_t>(L.v_codebook) % 16)
            return LVQ_ERR_INVALID_ARG;
    }
    if (!lvq::decode_supported(c->head_dim, S, cg, c->codebook_dtype == LVQ_BF16) ||
        c->head_dim > lvq::kMaxDecodeDim)
        return LVQ_ERR_UNSUPPORTED;
    // the index rows of one (b, h) are addressed with 32-bit byte offsets
    if ((int64_t)c->max_tokens * S > 0x7fffffff - 65536LL * S) return LVQ_ERR_UNSUPPORTED;
    // the header, then one block per (layer, b, h); n_layers single-layer
    // workspaces hold that
    const uint64_t per_layer = lvq::layer_block_bytes(c->batch, c->n_heads);
    const int64_t max_vq = max_vq_tokens(c, max_ctx_len, vq_len == nullptr);
    if (use_scratch) {
        workspace_bytes = lvq::kScratchBytes;
        for (int32_t l0 = 0; l0 < n_layers; l0 += lvq::kMaxLayersPerLaunch) {
            const int32_t nl = std::min<int32_t>(lvq::kMaxLayersPerLaunch, n_layers - l0);
            if (decode_plan(c, max_vq, nl).sp.n > 1 &&
                (workspace_bytes - lvq::kHeaderBytes) / per_layer < (uint64_t)(l0 + nl))
                return LVQ_ERR_WORKSPACE;
        }
        const hipError_t e = lvq::scratch_address(static_cast<hipStream_t>(stream), &workspace);
        if (e != hipSuccess) return LVQ_ERR_HIP;
    } else {
        if (!workspace || workspace_bytes < lvq::kHeaderBytes ||
            (workspace_bytes - lvq::kHeaderBytes) / per_layer < (uint64_t)n_layers)
            return LVQ_ERR_WORKSPACE;
        if (reinterpret_cast<uintptr_t>(workspace) % 256) return LVQ_ERR_INVALID_ARG;
    }

    const int64_t Hk = kv_heads(c);
    const size_t W = (size_t)c->n_sink + c->n_recent;
    for (int32_t l0 = 0; l0 < n_layers; l0 += lvq::kMaxLayersPerLaunch) {
        const int32_t nl = std::min<int32_t>(lvq::kMaxLayersPerLaunch, n_layers - l0);
        const Plan plan = decode_plan(c, max_vq, nl);
        if (plan.nh == 0) return LVQ_ERR_UNSUPPORTED;     // two heads per workgroup asked, not possible
        const Splits sp = plan.sp;
        const int32_t n_split = sp.n;
        if ((int64_t)n_split * c->batch * c->n_heads * nl > 0x7fffffff) return LVQ_ERR_UNSUPPORTED;
        const int64_t n_vq = n_split - sp.n_win;
        int64_t chunk = (max_vq + n_vq - 1) / n_vq;
        chunk = (chunk + 63) / 64 * 64;
        if (chunk < 64) chunk = 64;

        lvq::DecodeArgs a{};
        a.B = c->batch;
        a.H = c->n_heads;
        a.Hk = (int)Hk;
        a.q_per_kv = c->n_heads / a.Hk;
        a.d = c->head_dim;
        a.cg = cg;
        a.S = S;
        a.n_sink = c->n_sink;
        a.n_recent = c->n_recent;
        a.t_max = c->max_tokens;
        a.n_split = n_split;
        a.window_wg = sp.n_win;
        {
            const int64_t ranges = sp.n_win > 0 ? sp.n_win : n_split;
            a.win_per = (int)(((int64_t)W + ranges - 1) / ranges);
        }
        a.chunk = (int)chunk;
        // (the head-pair variant takes sequences in index order)
        a.by_length = plan.nh == 1 && n_split == 1 && nl == 1 && c->batch > 1 &&
                      c->batch <= lvq::kMaxOrderedBatch;
        a.cb_bf16 = c->codebook_dtype == LVQ_BF16;
        a.n_layers = nl;
        a.heads_per_wg = plan.nh;
        a.ctx_len = ctx_len;
        a.vq_len = vq_len;
        a.win_bstride = n_loops(c) * a.Hk * W * c->head_dim;
        a.scale_log2 = sm_scale * 1.4426950408889634f;
        a.blocks = static_cast<char *>(workspace) + lvq::kHeaderBytes + (size_t)l0 * per_layer;
        a.status = static_cast<uint32_t *>(workspace);
        a.max_polls = c->decode_poll_limit > 0 ? c->decode_poll_limit : kDefaultPolls;
        // loop step r reads the index rows of group r / Tc, codebook slice r
        // and window buffers of step r
        const size_t grp = (size_t)(loop_step / c->loop_steps) * c->batch * Hk * c->max_tokens * S;
        const size_t cbe = c->codebook_dtype == LVQ_BF16 ? 2 : 4;
        const size_t slice = (size_t)loop_step * Hk * S * LVQ_CODES * cg * cbe;
        const size_t wstep = (size_t)loop_step * Hk * W * c->head_dim;
        for (int32_t i = 0; i < nl; ++i) {
            const lvq_decode_layer &L = layers[l0 + i];
            lvq::DecodeLayer &d = a.layer[i];
            d.q = static_cast<const uint16_t *>(L.q);
            d.k_index = L.k_index + grp;
            d.v_index = L.v_index + grp;
            d.kcb_t = static_cast<const char *>(L.k_codebook) + slice;
            d.vcb_t = static_cast<const char *>(L.v_codebook) + slice;
            d.kwin_t = static_cast<const uint16_t *>(L.k_window) + wstep;
            d.vwin_t = static_cast<const uint16_t *>(L.v_window) + wstep;
            d.out = L.out;
        }
        const hipError_t e = lvq::launch_decode(a, static_cast<hipStream_t>(stream));
        if (e != hipSuccess) return LVQ_ERR_HIP;
    }
    return LVQ_OK;
}

}  // namespace

lvq_status lvq_decode_attn(const lvq_config *c, int32_t loop_step, const void *q,
                           const int32_t *ctx_len, const int32_t *vq_len,
                           int32_t max_ctx_len, const uint8_t *k_index,
                           const uint8_t *v_index, const void *k_codebook,
                           const void *v_codebook, const void *k_window,
                           const void *v_window, float sm_scale, void *workspace,
                           uint64_t workspace_bytes, float *out, void *stream) {
    const lvq_decode_layer layer{q, k_index, v_index, k_codebook, v_codebook, k_window, v_window, out};
    return decode_layers(c, 1, loop_step, &layer, ctx_len, vq_len, max_ctx_len, sm_scale, workspace,
                         workspace_bytes, stream);
}

lvq_status lvq_decode_attn_noalloc(const lvq_config *c, int32_t loop_step, const void *q,
                                   const int32_t *ctx_len, const int32_t *vq_len,
                                   int32_t max_ctx_len, const uint8_t *k_index,
                                   const uint8_t *v_index, const void *k_codebook,
                                   const void *v_codebook, const void *k_window,
                                   const void *v_window, float sm_scale, float *out,
                                   void *stream) {
    const lvq_decode_layer layer{q, k_index, v_index, k_codebook, v_codebook, k_window, v_window, out};
    return decode_layers(c, 1, loop_step, &layer, ctx_len, vq_len, max_ctx_len, sm_scale, nullptr, 0,
                         stream, true);
}

lvq_status lvq_decode_attn_layers(const lvq_config *c, int32_t n_layers, int32_t loop_step,
                                  const lvq_decode_layer *layers, const int32_t *ctx_len,
                                  const int32_t *vq_len, int32_t max_ctx_len, float sm_scale,
                                  void *workspace, uint64_t workspace_bytes, void *stream) {
    return decode_layers(c, n_layers, loop_step, layers, ctx_len, vq_len, max_ctx_len, sm_scale,
                         workspace, workspace_bytes, stream);
}

lvq_status lvq_decode_status(void *workspace, uint32_t *flags, int32_t clear, void *stream) {
    if (!workspace || !flags) return LVQ_ERR_INVALID_ARG;
    if (reinterpret_cast<uintptr_t>(workspace) % 256) return LVQ_ERR_INVALID_ARG;
    const hipStream_t st = static_cast<hipStream_t>(stream);
    uint32_t w = 0;
    if (hipStreamSynchronize(st) != hipSuccess) return LVQ_ERR_HIP;
    if (hipMemcpy(&w, workspace, sizeof w, hipMemcpyDeviceToHost) != hipSuccess) return LVQ_ERR_HIP;
    if (clear && w != 0) {
        const uint32_t zero = 0;
        if (hipMemcpy(workspace, &zero, sizeof zero, hipMemcpyHostToDevice) != hipSuccess)
            return LVQ_ERR_HIP;
    }
    *flags = w;
    return LVQ_OK;
}

int32_t lvq_decode_role(const lvq_config *c, int32_t n_layers, int32_t max_ctx_len,
                        int32_t workgroup, int32_t *layer, int32_t *seq, int32_t *head) {
    if (!config_ok(c) || n_layers < 1 || n_layers > lvq::kMaxLayersPerLaunch) return -1;
    if (max_ctx_len < 0 || max_ctx_len > c->max_tokens) return -1;
    const Plan plan = decode_plan(c, max_vq_tokens(c, max_ctx_len, true), n_layers);
    if (plan.nh == 0) return -1;
    const Splits sp = plan.sp;
    const int64_t hg = c->n_heads / plan.nh;            // head groups per sequence
    const int64_t total = (int64_t)sp.n * c->batch * hg * n_layers;
    if (workgroup < 0 || workgroup >= total) return -1;
    const lvq::WgRole r = lvq::decode_role((unsigned)workgroup, (unsigned)total, (unsigned)sp.n);
    const int64_t bh = (int64_t)c->batch * hg;
    if (layer) *layer = (int32_t)(r.group / bh);
    if (seq) *seq = (int32_t)(r.group % bh / hg);
    if (head) *head = (int32_t)(r.group % hg * plan.nh);
    return r.role;
}

}  // extern "C"
