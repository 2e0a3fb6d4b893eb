// LoopVQ decode attention for one loop step, gfx950.
//
// LoopVQ project page (mscheong01.github.io/loopvq), "Serving in SGLang --
// Attend from indices": at loop step t the keys and values of the VQ tokens
// are read from shared 8-bit indices through codebook slice t, and the result
// is merged with bf16 attention over the sink and recent tokens.
//
// One launch, grid (1 + n_split, H, B), 256 threads per workgroup:
//  * workgroup x = 0: dense attention of q over the valid bf16 window slots
//    of step t (online softmax per slot group, combined in LDS);
//  * workgroup x = s >= 1: VQ tokens [n_s + (s-1)*chunk, ...).  Instead of
//    dequantising keys, it builds the score table
//        T[j][k] = sm_scale * sum_c q[j*cg + c] * Bk_t[j][k][c]
//    in LDS once, so a token's score is sum_j T[j][idxK[n][j]] (S gathers).
//    Instead of dequantising values, it accumulates the softmax weight of
//    every token into a per-(sub-vector, code) histogram
//        W[j][k] += p_n   for k = idxV[n][j]
//    (LDS float atomics) and contracts once at the end:
//        o[j*cg + c] = sum_k W[j][k] * Bv_t[j][k][c].
//    Scores of a 1024-token tile are computed first, so the running maximum
//    only changes between tiles (W and l are rescaled then).
//  * every workgroup stores (m, l, o[d]) to the workspace and takes a ticket;
//    the last arrival of a (b, h) merges the partials (log-sum-exp) into out
//    and resets the ticket.
#include "kernels.h"

#include <math.h>

namespace lvq {
namespace {

constexpr int kThreads = 256;
constexpr int kTokPerThread = 4;
constexpr int kTile = kThreads * kTokPerThread;

__device__ __forceinline__ float bf16f(uint16_t b) { return __uint_as_float((uint32_t)b << 16); }

template <typename CB>
__device__ __forceinline__ float cb_at(const CB *p, int i);
template <>
__device__ __forceinline__ float cb_at<float>(const float *p, int i) { return p[i]; }
template <>
__device__ __forceinline__ float cb_at<uint16_t>(const uint16_t *p, int i) { return bf16f(p[i]); }

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

template <int S>
struct Row {
    uint32_t w[S / 4];
};

template <int S>
__device__ __forceinline__ Row<S> load_row(const uint8_t *p) {
    Row<S> r;
    if constexpr (S % 16 == 0) {
#pragma unroll
        for (int i = 0; i < S / 16; ++i) {
            const uint4 v = reinterpret_cast<const uint4 *>(p)[i];
            r.w[4 * i + 0] = v.x;
            r.w[4 * i + 1] = v.y;
            r.w[4 * i + 2] = v.z;
            r.w[4 * i + 3] = v.w;
        }
    } else {
        const uint2 v = *reinterpret_cast<const uint2 *>(p);
        r.w[0] = v.x;
        r.w[1] = v.y;
    }
    return r;
}

template <int S>
__device__ __forceinline__ int row_byte(const Row<S> &r, int j) {
    return (r.w[j >> 2] >> ((j & 3) * 8)) & 0xff;
}

// ---------------------------------------------------------------------------
// bf16 window workgroup: (m, l, o) over the valid slots of step t.
// ---------------------------------------------------------------------------
template <int D>
__device__ void window_part(const DecodeArgs &a, int b, int h, const Windows &w,
                            const float *qs, float *scratch, float *part) {
    constexpr int CH = D / 8;          // lanes per slot (8 channels each)
    constexpr int SPP = kThreads / CH; // slot groups
    const int tid = threadIdx.x;
    const int lane = tid % CH, sg = tid / CH;
    const int W = a.n_sink + a.n_recent;
    const size_t base = (((size_t)b * a.Tc + a.loop_step) * a.H + h) * (size_t)W * D;
    const uint16_t *kw = a.k_win + base;
    const uint16_t *vw = a.v_win + base;
    float qv[8];
#pragma unroll
    for (int i = 0; i < 8; ++i) qv[i] = qs[lane * 8 + i];
    float m = -INFINITY, l = 0.f, acc[8];
#pragma unroll
    for (int i = 0; i < 8; ++i) acc[i] = 0.f;
    for (int slot = sg; slot < W; slot += SPP) {
        if (!slot_valid(slot, w, a.n_sink, a.n_recent)) continue;  // uniform per slot group
        const uint4 kk = *reinterpret_cast<const uint4 *>(kw + (size_t)slot * D + lane * 8);
        const uint4 vv = *reinterpret_cast<const uint4 *>(vw + (size_t)slot * D + lane * 8);
        const uint32_t kwd[4] = {kk.x, kk.y, kk.z, kk.w};
        const uint32_t vwd[4] = {vv.x, vv.y, vv.z, vv.w};
        float dot = 0.f;
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            dot += qv[2 * i] * __uint_as_float(kwd[i] << 16);
            dot += qv[2 * i + 1] * __uint_as_float(kwd[i] & 0xffff0000u);
        }
#pragma unroll
        for (int off = CH / 2; off >= 1; off >>= 1) dot += __shfl_xor(dot, off);
        const float mn = fmaxf(m, dot);
        const float sc = __expf(m - mn);
        const float p = __expf(dot - mn);
        l = l * sc + p;
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            acc[2 * i] = acc[2 * i] * sc + p * __uint_as_float(vwd[i] << 16);
            acc[2 * i + 1] = acc[2 * i + 1] * sc + p * __uint_as_float(vwd[i] & 0xffff0000u);
        }
        m = mn;
    }
    // combine the slot groups: scratch[sg][0] = m, [1] = l, [2 + ch] = acc
    float *mine = scratch + sg * (D + 2);
    if (lane == 0) {
        mine[0] = m;
        mine[1] = l;
    }
#pragma unroll
    for (int i = 0; i < 8; ++i) mine[2 + lane * 8 + i] = acc[i];
    __syncthreads();
    float M = -INFINITY;
    for (int g = 0; g < SPP; ++g)
        if (scratch[g * (D + 2) + 1] > 0.f) M = fmaxf(M, scratch[g * (D + 2)]);
    for (int ch = tid; ch < D; ch += kThreads) {
        float o = 0.f;
        for (int g = 0; g < SPP; ++g) {
            const float *pg = scratch + g * (D + 2);
            if (pg[1] > 0.f) o += pg[2 + ch] * __expf(pg[0] - M);
        }
        part[2 + ch] = o;
    }
    if (tid == 0) {
        float lt = 0.f;
        for (int g = 0; g < SPP; ++g) {
            const float *pg = scratch + g * (D + 2);
            if (pg[1] > 0.f) lt += pg[1] * __expf(pg[0] - M);
        }
        part[0] = M;
        part[1] = lt;
    }
}

// ---------------------------------------------------------------------------
// VQ workgroup: score table + weight histogram over one split of VQ tokens.
// ---------------------------------------------------------------------------
template <int S, int CG, typename CB>
__device__ void vq_part(const DecodeArgs &a, int b, int h, int split, const Windows &w,
                        const float *qs, float *lut, float *hist, float *red, float *part) {
    constexpr int NT = S * 256;
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int vq_end = w.n_s + w.n_v;
    const int start = w.n_s + (split - 1) * a.chunk;
    const int end = min(start + a.chunk, vq_end);
    if (start >= end) {
        if (tid == 0) {
            part[0] = -INFINITY;
            part[1] = 0.f;
        }
        return;
    }
    const size_t slice = ((size_t)a.loop_step * a.H + h) * (size_t)NT * CG;
    const CB *kcb = static_cast<const CB *>(a.k_cb) + slice;
    const CB *vcb = static_cast<const CB *>(a.v_cb) + slice;

    // score table T[j][k] and zeroed histogram
    for (int e = tid; e < NT; e += kThreads) {
        const int j = e >> 8;
        const CB *row = kcb + (size_t)e * CG;
        float acc = 0.f;
#pragma unroll
        for (int c = 0; c < CG; ++c) acc += qs[j * CG + c] * cb_at(row, c);
        lut[e] = acc;
        hist[e] = 0.f;
    }
    __syncthreads();

    const size_t rows = ((size_t)b * a.H + h) * (size_t)a.t_max;
    const uint8_t *kidx = a.k_index + rows * S;
    const uint8_t *vidx = a.v_index + rows * S;
    float M = -INFINITY, lsum = 0.f;
    int parity = 0;
    for (int base = start; base < end; base += kTile) {
        Row<S> kr[kTokPerThread], vr[kTokPerThread];
        bool ok[kTokPerThread];
#pragma unroll
        for (int r = 0; r < kTokPerThread; ++r) {
            const int n = base + tid + r * kThreads;
            ok[r] = n < end;
            if (ok[r]) {
                kr[r] = load_row<S>(kidx + (size_t)n * S);
                vr[r] = load_row<S>(vidx + (size_t)n * S);
            }
        }
        float s[kTokPerThread];
        float tmax = -INFINITY;
#pragma unroll
        for (int r = 0; r < kTokPerThread; ++r) {
            float acc = 0.f;
            if (ok[r]) {
#pragma unroll
                for (int j = 0; j < S; ++j) acc += lut[j * 256 + row_byte<S>(kr[r], j)];
            }
            s[r] = ok[r] ? acc : -INFINITY;
            tmax = fmaxf(tmax, s[r]);
        }
        tmax = wave_max(tmax);
        if (lane == 0) red[parity * 4 + wave] = tmax;
        __syncthreads();
        tmax = fmaxf(fmaxf(red[parity * 4 + 0], red[parity * 4 + 1]),
                     fmaxf(red[parity * 4 + 2], red[parity * 4 + 3]));
        parity ^= 1;
        if (tmax > M) {  // uniform across the workgroup
            if (M != -INFINITY) {
                const float sc = __expf(M - tmax);
                for (int e = tid; e < NT; e += kThreads) hist[e] *= sc;
                lsum *= sc;
                __syncthreads();
            }
            M = tmax;
        }
#pragma unroll
        for (int r = 0; r < kTokPerThread; ++r) {
            if (ok[r]) {
                const float p = __expf(s[r] - M);
                lsum += p;
#pragma unroll
                for (int j = 0; j < S; ++j) atomicAdd(&hist[j * 256 + row_byte<S>(vr[r], j)], p);
            }
        }
    }
    __syncthreads();

    // o[j*CG + c] = sum_k W[j][k] * Bv_t[j][k][c]
    constexpr int TPJ = kThreads / S;   // threads per sub-vector
    {
        const int j = tid / TPJ, r = tid % TPJ;
        float acc[CG];
#pragma unroll
        for (int c = 0; c < CG; ++c) acc[c] = 0.f;
        for (int k = r; k < 256; k += TPJ) {
            const float wgt = hist[j * 256 + k];
            const CB *row = vcb + ((size_t)j * 256 + k) * CG;
#pragma unroll
            for (int c = 0; c < CG; ++c) acc[c] += wgt * cb_at(row, c);
        }
#pragma unroll
        for (int off = TPJ / 2; off >= 1; off >>= 1)
#pragma unroll
            for (int c = 0; c < CG; ++c) acc[c] += __shfl_xor(acc[c], off);
        if (r == 0) {
#pragma unroll
            for (int c = 0; c < CG; ++c) part[2 + j * CG + c] = acc[c];
        }
    }
    lsum = wave_sum(lsum);
    __syncthreads();
    if (lane == 0) red[wave] = lsum;
    __syncthreads();
    if (tid == 0) {
        part[0] = M;
        part[1] = red[0] + red[1] + red[2] + red[3];
    }
}

template <int S, int CG, typename CB>
__global__ __launch_bounds__(kThreads) void decode_kernel(DecodeArgs a) {
    constexpr int D = S * CG;
    __shared__ float smem[2 * S * 256];
    __shared__ float qs[D];
    __shared__ float red[8];
    __shared__ int is_last;

    const int split = blockIdx.x, h = blockIdx.y, b = blockIdx.z;
    const int tid = threadIdx.x;
    const Windows w = seq_windows(a, b);
    float *part = a.partials + (((size_t)b * a.H + h) * kSlots + split) * (D + 2);

    for (int i = tid; i < D; i += kThreads)
        qs[i] = bf16f(a.q[((size_t)b * a.H + h) * D + i]) * a.sm_scale;
    __syncthreads();

    if (split == 0)
        window_part<D>(a, b, h, w, qs, smem, part);
    else
        vq_part<S, CG, CB>(a, b, h, split, w, qs, smem, smem + S * 256, red, part);

    // publish the partial, then count arrivals; the last one merges
    __threadfence();
    __syncthreads();
    if (tid == 0) {
        const unsigned prev = atomicAdd(&a.tickets[(size_t)b * a.H + h], 1u);
        is_last = prev == (unsigned)a.n_split;
    }
    __syncthreads();
    if (!is_last) return;
    __threadfence();

    const float *pb = a.partials + ((size_t)b * a.H + h) * kSlots * (D + 2);
    const int nslots = a.n_split + 1;
    float M = -INFINITY;
    for (int i = 0; i < nslots; ++i)
        if (pb[i * (D + 2) + 1] > 0.f) M = fmaxf(M, pb[i * (D + 2)]);
    float den = 0.f;
    for (int i = 0; i < nslots; ++i) {
        const float li = pb[i * (D + 2) + 1];
        if (li > 0.f) den += li * __expf(pb[i * (D + 2)] - M);
    }
    for (int ch = tid; ch < D; ch += kThreads) {
        float num = 0.f;
        for (int i = 0; i < nslots; ++i) {
            const float *pi = pb + i * (D + 2);
            if (pi[1] > 0.f) num += pi[2 + ch] * __expf(pi[0] - M);
        }
        a.out[((size_t)b * a.H + h) * D + ch] = den > 0.f ? num / den : 0.f;
    }
    if (tid == 0) a.tickets[(size_t)b * a.H + h] = 0u;
}

template <int S, int CG>
hipError_t launch_sc(const DecodeArgs &a, hipStream_t st) {
    const dim3 grid(a.n_split + 1, a.H, a.B);
    if (a.cb_bf16)
        hipLaunchKernelGGL((decode_kernel<S, CG, uint16_t>), grid, dim3(kThreads), 0, st, a);
    else
        hipLaunchKernelGGL((decode_kernel<S, CG, float>), grid, dim3(kThreads), 0, st, a);
    return hipGetLastError();
}

}  // namespace

bool decode_supported(int d, int S, int cg) {
    if (d % 8 != 0 || d > 256 || d < 16) return false;
    if (S != 8 && S != 16 && S != 32 && S != 64) return false;
    if (cg != 2 && cg != 4 && cg != 8) return false;
    return S * cg == d;
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
    LVQ_CASE(32, 8)
    LVQ_CASE(64, 2)
    LVQ_CASE(64, 4)
#undef LVQ_CASE
    return hipErrorInvalidValue;
}

}  // namespace lvq
