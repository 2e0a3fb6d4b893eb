// Test infrastructure: stand-ins for the kernel launchers and the two HIP
// runtime calls of the library's host code, so that loopvq_host.cpp can be
// built for the host alone (with address and undefined-behaviour sanitizers)
// and driven through its C ABI without a GPU.  A "launch" checks the
// invariants of the arguments the host code assembled and counts itself; it
// never touches the pointers.  The shape predicates follow the supported
// shapes stated in include/loopvq.h.
#include <hip/hip_runtime.h>

#include <cstdint>
#include <cstring>

#include "kernels.h"

namespace {
int g_decode_launches = 0, g_encode_launches = 0, g_bad_args = 0;
alignas(256) unsigned char g_scratch[256];

bool bad(bool cond) {
    if (cond) ++g_bad_args;
    return cond;
}
}  // namespace

namespace lvq {

bool decode_supported(int d, int S, int cg, int cb_bf16) {
    const bool s_ok = S == 8 || S == 16 || S == 32 || S == 64;
    const bool cg_ok = cg == 2 || cg == 4 || cg == 8;
    return s_ok && cg_ok && S * cg == d && S * cg * (cb_bf16 ? 2 : 4) <= 256 && d <= kMaxDecodeDim;
}

bool encode_supported(int G, int cg, int S, int cb_bf16) {
    if (G != 8 && G != 16 && G != 32) return false;
    if (cg != 2 && cg != 4 && cg != 8) return false;
    if (cg > G || S % 4 != 0) return false;
    return cb_bf16 || G <= 16;
}

hipError_t launch_decode(const DecodeArgs &a, hipStream_t) {
    ++g_decode_launches;
    bool fail = false;
    fail |= bad(a.n_split < 1 || a.n_split > kMaxSplits);
    fail |= bad(a.window_wg < 0 || (a.window_wg > 0 && a.window_wg >= a.n_split));
    fail |= bad(a.chunk < 64 || a.chunk % 64 != 0);
    {
        // the window ranges cover [0, W) and index arithmetic stays in 32 bits
        const int64_t W = (int64_t)a.n_sink + a.n_recent;
        const int64_t ranges = a.window_wg > 0 ? a.window_wg : a.n_split;
        fail |= bad(a.win_per < 1 || ranges * a.win_per < W || (int64_t)a.n_split * a.win_per > 0x7fffffff);
    }
    fail |= bad(a.n_layers < 1 || a.n_layers > kMaxLayersPerLaunch);
    fail |= bad(a.Hk < 1 || a.q_per_kv < 1 || a.Hk * a.q_per_kv != a.H);
    fail |= bad(a.S * a.cg != a.d || a.t_max < 1 || a.max_polls < 1);
    fail |= bad(!a.ctx_len || !a.blocks || !a.status);
    fail |= bad(a.by_length && (a.n_split != 1 || a.n_layers != 1 || a.B < 2 || a.B > kMaxOrderedBatch));
    // head pairs: the kernel's variant for S = 32, cg = 4, bf16, d = 128, one
    // layer, two query heads of one KV head, merging through window
    // workgroups (or no merge)
    fail |= bad(a.heads_per_wg != 1 && a.heads_per_wg != 2);
    fail |= bad(a.heads_per_wg == 2 &&
                (a.S != 32 || a.cg != 4 || !a.cb_bf16 || a.d != 128 || a.n_layers != 1 || a.by_length ||
                 a.q_per_kv % 2 != 0 || (a.n_split > 1 && a.window_wg == 0)));
    for (int l = 0; l < a.n_layers; ++l) {
        const DecodeLayer &L = a.layer[l];
        fail |= bad(!L.q || !L.k_index || !L.v_index || !L.kcb_t || !L.vcb_t || !L.kwin_t || !L.vwin_t || !L.out);
    }
    return fail ? hipErrorInvalidValue : hipSuccess;
}

hipError_t launch_encode(const EncodeArgs &a, hipStream_t) {
    ++g_encode_launches;
    bool fail = false;
    fail |= bad(a.n_tokens < 1 || a.G != a.Tc * a.cg || a.S * a.cg != a.d);
    fail |= bad(!a.x || !a.cb || !a.index || a.n_tensors < 1 || a.n_tensors > 2);
    fail |= bad(a.n_tensors == 2 && (!a.x_b || !a.cb_b || !a.index_b));
    fail |= bad(a.first_token < 0 || a.first_token + a.n_tokens > a.t_max);
    return fail ? hipErrorInvalidValue : hipSuccess;
}

hipError_t scratch_address(hipStream_t, void **addr) {
    *addr = g_scratch;
    return hipSuccess;
}

}  // namespace lvq

extern "C" {
hipError_t hipStreamSynchronize(hipStream_t) { return hipSuccess; }
hipError_t hipMemcpy(void *dst, const void *src, size_t n, hipMemcpyKind) {
    std::memcpy(dst, src, n);
    return hipSuccess;
}
int lvq_stub_counts(int which) {
    return which == 0 ? g_decode_launches : which == 1 ? g_encode_launches : g_bad_args;
}
}
