// LoopVQ decode attention for one loop step, gfx950.
//
// LoopVQ project page (mscheong01.github.io/loopvq), "Serving in SGLang --
// Attend from indices": at loop step t the keys and values of the VQ tokens
// are read from shared 8-bit indices through codebook slice t, and the result
// is merged with bf16 attention over the sink and recent tokens.
//
// Two launches per call:
//  decode_main, grid (n_split, H, B), 512 threads.  Workgroup s of (b, h)
//    takes VQ tokens [n_s + s*chunk, ...) and window slots
//    [s*W/n_split, (s+1)*W/n_split).  It stages two tables in LDS:
//      T[j][k]  = log2(e) * sm_scale * sum_c q[j*cg + c] * Bk_t[j][k][c]  (fp32)
//      V[j][k]  = Bv_t[j][k][0..cg)  (fp16 for bf16 codebooks, else fp32)
//    A token's score is sum_j T[j][idxK[n][j]] (S gathers) and its value
//    row is gathered as V[j][idxV[n][j]] (S gathers of cg entries).
//    R = S/8 lanes share a token, each owning 8 sub-vectors (8*cg output
//    channels); every wave keeps its own running max, weight sum and
//    accumulators (online softmax, base 2), so tiles need no barrier.
//    Token weights p = 2^(s - m) enter the value sum as fp16 p * 2^14 through
//    v_dot2_f32_f16, and the weight sum adds the same rounded values, so the
//    result is an exact weighted average with weights perturbed by at most
//    2^-11 relative.  Waves combine in LDS; the workgroup stores (m, l, o).
//  decode_merge, grid (H, B): log-sum-exp merge of the n_split partials.
// The kernel boundary orders the partial stores before the merge's loads;
// no device-scope fence is needed.
#include "kernels.h"

#include <math.h>

#include <type_traits>

namespace lvq {
namespace {

constexpr int kThreads = 512;
constexpr int kWaves = kThreads / 64;
constexpr int kUnroll = 4;                     // token passes in flight per wave
constexpr float kLog2e = 1.4426950408889634f;
constexpr float kPScale = 16384.f;             // p' = p * 2^14 (normal in fp16 down to p ~ 4e-9)
constexpr int kLdsLimit = 160 * 1024;

typedef _Float16 half2_t __attribute__((ext_vector_type(2)));

__device__ __forceinline__ float bf16f(uint16_t b) { return __uint_as_float((uint32_t)b << 16); }
__device__ __forceinline__ float bf16lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf16hi(uint32_t w) { return __uint_as_float(w & 0xffff0000u); }

template <typename CB>
__device__ __forceinline__ float cb_at(const CB *p, int i);
template <>
__device__ __forceinline__ float cb_at<float>(const float *p, int i) { return p[i]; }
template <>
__device__ __forceinline__ float cb_at<uint16_t>(const uint16_t *p, int i) { return bf16f(p[i]); }

template <int S, int CG, typename CB>
struct Shape {
    static constexpr int D = S * CG;
    static constexpr int R = S / 8;            // lanes per token
    static constexpr int TPW = 64 / R;         // tokens per wave pass
    static constexpr int CL = 8 * CG;          // output channels per lane
    static constexpr bool kF16V = std::is_same<CB, uint16_t>::value;
    static constexpr int VB = kF16V ? 2 : 4;   // bytes per value-table entry
    static constexpr int kLut = S * 256;       // floats
    static constexpr int kVtabWords = S * 256 * CG * VB / 4;
    static constexpr int kScratch = kWaves * (D + 2);
    static constexpr int kLds = 4 * (kLut + kVtabWords + kScratch + D) + 64;
};

struct Windows {
    int L, n_s, n_v;
};

__device__ __forceinline__ Windows seq_windows(const DecodeArgs &a, int b) {
    int L = a.ctx_len[b];
    L = max(0, (int)min((int64_t)L, a.t_max));
    const int n_s = min(L, a.n_sink);
    int n_v;
    if (a.vq_len) {
        n_v = max(0, min(a.vq_len[b], L - n_s));
    } else {
        n_v = max(0, L - a.n_sink - a.n_recent);
    }
    return {L, n_s, n_v};
}

// Does window slot `slot` hold a token of the current sink/recent windows?
// Recent token p sits in slot n_sink + ((p - n_sink) mod n_recent); the slot
// holds the newest such p below L.
__device__ __forceinline__ bool slot_valid(int slot, const Windows &w, int n_sink, int n_recent) {
    if (slot < n_sink) return slot < w.n_s;
    if (w.L <= n_sink) return false;
    const int r = slot - n_sink;
    const int A = w.L - 1 - n_sink;
    if (r > A) return false;
    const int pos = n_sink + r + n_recent * ((A - r) / n_recent);
    return pos >= w.n_s + w.n_v;
}

__device__ __forceinline__ float wave_max(float v) {
#pragma unroll
    for (int off = 32; off >= 1; off >>= 1) v = fmaxf(v, __shfl_xor(v, off));
    return v;
}
__device__ __forceinline__ float wave_sum(float v) {
#pragma unroll
    for (int off = 32; off >= 1; off >>= 1) v += __shfl_xor(v, off);
    return v;
}

// Per-wave online-softmax state: running max m (base 2), weight sum l (scaled
// by 2^14; lanes with r == 0 count each token once) and accumulators.
template <int NACC>
struct Online {
    float m = -INFINITY;
    float l = 0.f;
    float acc[NACC];

    __device__ __forceinline__ void init() {
#pragma unroll
        for (int i = 0; i < NACC; ++i) acc[i] = 0.f;
    }
    // raise the running max to at least `mx` (wave-uniform)
    __device__ __forceinline__ void raise(float mx) {
        if (mx > m) {
            const float sc = exp2f(m - mx);   // 0 when m = -inf
            l *= sc;
#pragma unroll
            for (int i = 0; i < NACC; ++i) acc[i] *= sc;
            m = mx;
        }
    }
};

// ---------------------------------------------------------------------------
// Table staging: score table and value table of (h, loop step t) into LDS.
// ---------------------------------------------------------------------------
template <int S, int CG, typename CB>
__device__ __forceinline__ void stage_tables(const DecodeArgs &a, int h, const float *qs,
                                             float *lut, uint32_t *vtab) {
    using Sh = Shape<S, CG, CB>;
    const size_t slice = ((size_t)a.loop_step * a.H + h) * (size_t)Sh::kLut * CG;
    const CB *kcb = static_cast<const CB *>(a.k_cb) + slice;
    const CB *vcb = static_cast<const CB *>(a.v_cb) + slice;
    const int tid = threadIdx.x;
    // T[e], e = j*256 + k: dot of q[j*cg ..] with codeword entries (contiguous)
    constexpr int PER = Sh::kLut / kThreads;
    static_assert(Sh::kLut % kThreads == 0, "score table must tile the workgroup");
    float cw[PER][CG];
#pragma unroll
    for (int u = 0; u < PER; ++u) {
        const int e = tid + u * kThreads;
#pragma unroll
        for (int c = 0; c < CG; ++c) cw[u][c] = cb_at(kcb + (size_t)e * CG, c);
    }
#pragma unroll
    for (int u = 0; u < PER; ++u) {
        const int e = tid + u * kThreads;
        const int j = e >> 8;
        float acc = 0.f;
#pragma unroll
        for (int c = 0; c < CG; ++c) acc += qs[j * CG + c] * cw[u][c];
        lut[e] = acc;
    }
    // value table: same entry order, converted to fp16 (bf16 codebooks) or
    // copied (fp32 codebooks); 16 bytes of source per step
    if constexpr (Sh::kF16V) {
        constexpr int N8 = Sh::kLut * CG / 8;          // groups of 8 bf16
        const uint4 *src = reinterpret_cast<const uint4 *>(vcb);
        uint4 *dst = reinterpret_cast<uint4 *>(vtab);
        for (int g = tid; g < N8; g += kThreads) {
            const uint4 v = src[g];
            const uint32_t w[4] = {v.x, v.y, v.z, v.w};
            uint32_t o[4];
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const half2_t hp = {(_Float16)bf16lo(w[i]), (_Float16)bf16hi(w[i])};
                o[i] = __builtin_bit_cast(uint32_t, hp);
            }
            dst[g] = make_uint4(o[0], o[1], o[2], o[3]);
        }
    } else {
        constexpr int N4 = Sh::kLut * CG / 4;          // groups of 4 fp32
        const uint4 *src = reinterpret_cast<const uint4 *>(vcb);
        uint4 *dst = reinterpret_cast<uint4 *>(vtab);
        for (int g = tid; g < N4; g += kThreads) dst[g] = src[g];
    }
}

// ---------------------------------------------------------------------------
// Dense bf16 window slots [s0, s1): R lanes per slot, each owning CL channels.
// ---------------------------------------------------------------------------
template <int S, int CG, typename CB, typename OnlineT>
__device__ __forceinline__ void window_slots(const DecodeArgs &a, int b, int h, const Windows &w,
                                             int s0, int s1, const float *qs, OnlineT &st) {
    using Sh = Shape<S, CG, CB>;
    constexpr int D = Sh::D, R = Sh::R, TPW = Sh::TPW, CL = Sh::CL;
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const int r = lane % R, tg = lane / R;
    const int W = a.n_sink + a.n_recent;
    const size_t base = (((size_t)b * a.Tc + a.loop_step) * a.H + h) * (size_t)W * D + r * CL;
    const uint16_t *kw = a.k_win + base;
    const uint16_t *vw = a.v_win + base;
    for (int sb = s0 + wave * TPW; sb < s1; sb += kWaves * TPW) {   // wave-uniform loop
        const int slot = sb + tg;
        const bool ok = slot < s1 && slot_valid(slot, w, a.n_sink, a.n_recent);
        float dot = 0.f;
        uint32_t vv[CL / 2];
        if (ok) {
            const uint4 *kp = reinterpret_cast<const uint4 *>(kw + (size_t)slot * D);
            const uint4 *vp = reinterpret_cast<const uint4 *>(vw + (size_t)slot * D);
#pragma unroll
            for (int i = 0; i < CL / 8; ++i) {
                const uint4 kk = kp[i];
                const uint4 v4 = vp[i];
                const uint32_t kwd[4] = {kk.x, kk.y, kk.z, kk.w};
                vv[4 * i + 0] = v4.x;
                vv[4 * i + 1] = v4.y;
                vv[4 * i + 2] = v4.z;
                vv[4 * i + 3] = v4.w;
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    dot += qs[r * CL + 8 * i + 2 * e] * bf16lo(kwd[e]);
                    dot += qs[r * CL + 8 * i + 2 * e + 1] * bf16hi(kwd[e]);
                }
            }
        }
#pragma unroll
        for (int off = 1; off < R; off <<= 1) dot += __shfl_xor(dot, off);
        const float s = ok ? dot : -INFINITY;
        const float mx = wave_max(s);
        if (mx == -INFINITY) continue;
        st.raise(mx);
        if (ok) {
            const float p = exp2f(s - st.m) * kPScale;
            if (r == 0) st.l += p;
#pragma unroll
            for (int i = 0; i < CL / 2; ++i) {
                st.acc[2 * i] += p * bf16lo(vv[i]);
                st.acc[2 * i + 1] += p * bf16hi(vv[i]);
            }
        }
    }
}

template <int S>
__device__ __forceinline__ int byte_of(const uint2 &w, int jj) {
    return ((jj < 4 ? w.x : w.y) >> ((jj & 3) * 8)) & 0xff;
}

// ---------------------------------------------------------------------------
// VQ tokens [t0, t1).
// ---------------------------------------------------------------------------
template <int S, int CG, typename CB, typename OnlineT>
__device__ __forceinline__ void vq_tokens(const DecodeArgs &a, int b, int h, int t0, int t1,
                                          const float *lut, const uint32_t *vtab, OnlineT &st) {
    using Sh = Shape<S, CG, CB>;
    constexpr int R = Sh::R, TPW = Sh::TPW;
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const int r = lane % R, tg = lane / R;
    const size_t rows = ((size_t)b * a.H + h) * (size_t)a.t_max;
    const uint8_t *kidx = a.k_index + rows * S + 8 * r;
    const uint8_t *vidx = a.v_index + rows * S + 8 * r;
    const float *lut_r = lut + r * 8 * 256;
    constexpr int VW = CG * Sh::VB / 4;                 // 32-bit words per value entry
    const uint32_t *vt_r = vtab + (size_t)r * 8 * 256 * VW;
    constexpr int STEP = kWaves * TPW;                   // tokens per pass of the workgroup

    for (int base = t0 + wave * TPW; base < t1; base += STEP * kUnroll) {   // wave-uniform
        uint2 kr[kUnroll], vr[kUnroll];
        bool ok[kUnroll];
#pragma unroll
        for (int u = 0; u < kUnroll; ++u) {
            const int n = base + u * STEP + tg;
            ok[u] = n < t1;
            if (ok[u]) {
                kr[u] = *reinterpret_cast<const uint2 *>(kidx + (size_t)n * S);
                vr[u] = *reinterpret_cast<const uint2 *>(vidx + (size_t)n * S);
            } else {
                kr[u] = make_uint2(0, 0);
                vr[u] = make_uint2(0, 0);
            }
        }
        float s[kUnroll];
        float mx = -INFINITY;
#pragma unroll
        for (int u = 0; u < kUnroll; ++u) {
            float acc = 0.f;
#pragma unroll
            for (int jj = 0; jj < 8; ++jj) acc += lut_r[jj * 256 + byte_of<S>(kr[u], jj)];
#pragma unroll
            for (int off = 1; off < R; off <<= 1) acc += __shfl_xor(acc, off);
            s[u] = ok[u] ? acc : -INFINITY;
            mx = fmaxf(mx, s[u]);
        }
        st.raise(wave_max(mx));
#pragma unroll
        for (int u = 0; u < kUnroll; ++u) {
            if (!ok[u]) continue;
            if constexpr (Sh::kF16V) {
                const _Float16 ph = (_Float16)(exp2f(s[u] - st.m) * kPScale);
                if (r == 0) st.l += (float)ph;
                const half2_t plo = {ph, (_Float16)0.f};
                const half2_t phi = {(_Float16)0.f, ph};
#pragma unroll
                for (int jj = 0; jj < 8; ++jj) {
                    const uint32_t *e = vt_r + (jj * 256 + byte_of<S>(vr[u], jj)) * VW;
                    uint32_t wv[VW];
                    if constexpr (VW == 1) {
                        wv[0] = e[0];
                    } else {
#pragma unroll
                        for (int i = 0; i < VW; i += 2) {
                            const uint2 t = *reinterpret_cast<const uint2 *>(e + i);
                            wv[i] = t.x;
                            wv[i + 1] = t.y;
                        }
                    }
#pragma unroll
                    for (int i = 0; i < VW; ++i) {
                        const half2_t hv = __builtin_bit_cast(half2_t, wv[i]);
                        st.acc[jj * CG + 2 * i] = __builtin_amdgcn_fdot2(hv, plo, st.acc[jj * CG + 2 * i], false);
                        st.acc[jj * CG + 2 * i + 1] =
                            __builtin_amdgcn_fdot2(hv, phi, st.acc[jj * CG + 2 * i + 1], false);
                    }
                }
            } else {
                const float p = exp2f(s[u] - st.m) * kPScale;
                if (r == 0) st.l += p;
#pragma unroll
                for (int jj = 0; jj < 8; ++jj) {
                    const float *e = reinterpret_cast<const float *>(vt_r) +
                                     (jj * 256 + byte_of<S>(vr[u], jj)) * CG;
#pragma unroll
                    for (int c = 0; c < CG; ++c) st.acc[jj * CG + c] += p * e[c];
                }
            }
        }
    }
}

template <int S, int CG, typename CB>
__global__ __launch_bounds__(kThreads) void decode_main(DecodeArgs a) {
    using Sh = Shape<S, CG, CB>;
    constexpr int D = Sh::D, R = Sh::R, CL = Sh::CL;
    static_assert(Sh::kLds <= kLdsLimit, "LDS budget");
    __shared__ float lut[Sh::kLut];
    __shared__ __align__(16) uint32_t vtab[Sh::kVtabWords];
    __shared__ float scratch[Sh::kScratch];
    __shared__ float qs[D];

    const int split = blockIdx.x, h = blockIdx.y, b = blockIdx.z;
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const Windows w = seq_windows(a, b);
    const int t0 = w.n_s + split * a.chunk;
    const int t1 = min(t0 + a.chunk, w.n_s + w.n_v);
    const int W = a.n_sink + a.n_recent;
    const int s0 = (int)((int64_t)W * split / a.n_split);
    const int s1 = (int)((int64_t)W * (split + 1) / a.n_split);

    for (int i = tid; i < D; i += kThreads)
        qs[i] = bf16f(a.q[((size_t)b * a.H + h) * D + i]) * (a.sm_scale * kLog2e);
    __syncthreads();
    if (t0 < t1) stage_tables<S, CG, CB>(a, h, qs, lut, vtab);
    __syncthreads();

    Online<CL> st;
    st.init();
    window_slots<S, CG, CB>(a, b, h, w, s0, s1, qs, st);
    if (t0 < t1) vq_tokens<S, CG, CB>(a, b, h, t0, t1, lut, vtab, st);

    // combine the lanes of the wave that own the same channels, then the waves
#pragma unroll
    for (int off = R; off < 64; off <<= 1)
#pragma unroll
        for (int i = 0; i < CL; ++i) st.acc[i] += __shfl_xor(st.acc[i], off);
    const float lw = wave_sum(st.l);
    float *mine = scratch + wave * (D + 2);
    if (lane < R) {
#pragma unroll
        for (int i = 0; i < CL; ++i) mine[2 + lane * CL + i] = st.acc[i];
    }
    if (lane == 0) {
        mine[0] = st.m;
        mine[1] = lw;
    }
    __syncthreads();
    float *part = a.partials + (((size_t)b * a.H + h) * kSlots + split) * (D + 2);
    float M = -INFINITY;
#pragma unroll
    for (int v = 0; v < kWaves; ++v)
        if (scratch[v * (D + 2) + 1] > 0.f) M = fmaxf(M, scratch[v * (D + 2)]);
    for (int ch = tid; ch < D; ch += kThreads) {
        float o = 0.f;
#pragma unroll
        for (int v = 0; v < kWaves; ++v) {
            const float *pv = scratch + v * (D + 2);
            if (pv[1] > 0.f) o += pv[2 + ch] * exp2f(pv[0] - M);
        }
        part[2 + ch] = o;
    }
    if (tid == 0) {
        float lt = 0.f;
#pragma unroll
        for (int v = 0; v < kWaves; ++v) {
            const float *pv = scratch + v * (D + 2);
            if (pv[1] > 0.f) lt += pv[1] * exp2f(pv[0] - M);
        }
        part[0] = M;
        part[1] = lt;
    }
}

// Log-sum-exp merge of the n_split partials of (b, h) into out.
template <int D>
__global__ __launch_bounds__(256) void decode_merge(DecodeArgs a) {
    __shared__ float ml[2 * kMaxSplits];
    const int h = blockIdx.x, b = blockIdx.y, tid = threadIdx.x;
    const float *pb = a.partials + ((size_t)b * a.H + h) * kSlots * (D + 2);
    const int n = a.n_split;
    for (int i = tid; i < n; i += blockDim.x) {
        ml[2 * i] = pb[i * (D + 2)];
        ml[2 * i + 1] = pb[i * (D + 2) + 1];
    }
    __syncthreads();
    float M = -INFINITY;
    for (int i = 0; i < n; ++i)
        if (ml[2 * i + 1] > 0.f) M = fmaxf(M, ml[2 * i]);
    float den = 0.f;
    for (int i = 0; i < n; ++i)
        if (ml[2 * i + 1] > 0.f) den += ml[2 * i + 1] * exp2f(ml[2 * i] - M);
    for (int ch = tid; ch < D; ch += blockDim.x) {
        float num = 0.f;
#pragma unroll 8
        for (int i = 0; i < n; ++i)
            if (ml[2 * i + 1] > 0.f) num += pb[i * (D + 2) + 2 + ch] * exp2f(ml[2 * i] - M);
        a.out[((size_t)b * a.H + h) * D + ch] = den > 0.f ? num / den : 0.f;
    }
}

template <int S, int CG, typename CB>
constexpr bool fits() {
    return Shape<S, CG, CB>::kLds <= kLdsLimit;
}

template <int S, int CG>
hipError_t launch_sc(const DecodeArgs &a, hipStream_t st) {
    const dim3 grid(a.n_split, a.H, a.B);
    if (a.cb_bf16) {
        if constexpr (fits<S, CG, uint16_t>())
            hipLaunchKernelGGL((decode_main<S, CG, uint16_t>), grid, dim3(kThreads), 0, st, a);
        else
            return hipErrorInvalidValue;
    } else {
        if constexpr (fits<S, CG, float>())
            hipLaunchKernelGGL((decode_main<S, CG, float>), grid, dim3(kThreads), 0, st, a);
        else
            return hipErrorInvalidValue;
    }
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    hipLaunchKernelGGL((decode_merge<S * CG>), dim3(a.H, a.B), dim3(S * CG < 256 ? S * CG : 256), 0,
                       st, a);
    return hipGetLastError();
}

}  // namespace

bool decode_supported(int d, int S, int cg, int cb_bf16) {
#define LVQ_FIT(S_, CG_) \
    if (S == S_ && cg == CG_) return cb_bf16 ? fits<S_, CG_, uint16_t>() : fits<S_, CG_, float>();
    if (S * cg != d) return false;
    LVQ_FIT(8, 2)
    LVQ_FIT(8, 4)
    LVQ_FIT(8, 8)
    LVQ_FIT(16, 2)
    LVQ_FIT(16, 4)
    LVQ_FIT(16, 8)
    LVQ_FIT(32, 2)
    LVQ_FIT(32, 4)
    LVQ_FIT(64, 2)
#undef LVQ_FIT
    return false;
}

hipError_t launch_decode(const DecodeArgs &a, hipStream_t st) {
#define LVQ_CASE(S_, CG_) \
    if (a.S == S_ && a.cg == CG_) return launch_sc<S_, CG_>(a, st);
    LVQ_CASE(8, 2)
    LVQ_CASE(8, 4)
    LVQ_CASE(8, 8)
    LVQ_CASE(16, 2)
    LVQ_CASE(16, 4)
    LVQ_CASE(16, 8)
    LVQ_CASE(32, 2)
    LVQ_CASE(32, 4)
    LVQ_CASE(64, 2)
#undef LVQ_CASE
    return hipErrorInvalidValue;
}

}  // namespace lvq
