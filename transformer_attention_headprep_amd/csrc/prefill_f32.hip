// prefill_f32.hip -- f32 attention of whole sequences on the vector ALUs.
//
// softmax(q k^T scale [+ causal mask, bottom-right when there are more keys than
// queries]) v (gizml:netops reference page, Functions > attention) without a score matrix: keys go in tiles of 32 through LDS and each
// query row keeps a running maximum m, sum l and output a, rescaled by
// c = e^(m_old - m_new) when the maximum moves (the blocked online softmax that
// page describes for its own f32 kernel).  One lane owns one query row, so the q
// prologue (HeadPrep of q: RMS, weight, split-half turn) runs entirely in that
// lane's registers when half is 0 or d/2; other halves are prepped beforehand.
// This path serves f32 operands; it is exact f32 FMA arithmetic, not bit-identical
// to any other order.
#include "common.h"
#include "kernels.h"

namespace attn {
namespace {

constexpr int kRows = 64;   // query rows per block (one wave)
constexpr int kKeys = 32;   // keys per LDS tile

template <int D, bool CAUSAL, bool PREP>
__global__ __launch_bounds__(kRows) void prefill_f32_kernel(const PrefillLaunch p) {
    __shared__ float4 ks[kKeys * D / 4];
    __shared__ float4 vs[kKeys * D / 4];

    const int b = blockIdx.z, h = blockIdx.y;
    const int qtile = gridDim.x - 1 - blockIdx.x;         // longest causal rows first
    const int64_t r = (int64_t)qtile * kRows + threadIdx.x;
    const bool row_ok = r < p.seq;
    // query r sits at key position r + qoff and table row first + r; with per-sequence
    // lengths, at past[b] + r over keys 0 .. past[b] + seq - 1 (NaN rows when past[b]
    // lies outside [0, pos0])
    int64_t tk = p.tk, qoff = p.tk - p.seq, first = p.pos0;
    bool bad_seq = false;
    if (p.past) {
        const int v = p.past[b];
        bad_seq = v < 0 || v > p.pos0;
        qoff = first = bad_seq ? 0 : v;
        tk = qoff + p.seq;
    }
    const int g = h / (p.hq / p.hkv);
    const float *qbase = static_cast<const float *>(p.q) + b * p.q_bs + (row_ok ? r : 0) * p.q_rs + h * D;

    float q[D];
#pragma unroll
    for (int e = 0; e < D; e += 4) {
        const float4 t = row_ok ? *reinterpret_cast<const float4 *>(qbase + e) : make_float4(0, 0, 0, 0);
        q[e] = t.x; q[e + 1] = t.y; q[e + 2] = t.z; q[e + 3] = t.w;
    }
    if constexpr (PREP) {
        float ss = 0.f;
#pragma unroll
        for (int e = 0; e < D; ++e) ss += q[e] * q[e];
        const float inv = 1.0f / __builtin_sqrtf(ss * (1.0f / D) + p.eps);
#pragma unroll
        for (int e = 0; e < D; ++e) q[e] = q[e] * inv * p.qw[e];
        if (p.half > 0 && row_ok) {   // half = D/2 (other halves are prepped beforehand)
            const float *cr = p.cos + (first + r) * (D / 2);
            const float *sr = p.sin + (first + r) * (D / 2);
#pragma unroll
            for (int e = 0; e < D / 2; ++e) {
                const float a = q[e], bb = q[e + D / 2];
                q[e] = a * cr[e] - bb * sr[e];
                q[e + D / 2] = bb * cr[e] + a * sr[e];
            }
        }
    }
    const float C = p.scale * kLog2e;   // scores in base-2 units

    float m = -INFINITY, l = 0.f;
    float o[D];
#pragma unroll
    for (int e = 0; e < D; ++e) o[e] = 0.f;

    const int64_t last_key = CAUSAL ? min<int64_t>(tk - 1, (int64_t)qtile * kRows + kRows - 1 + qoff) : tk - 1;
    const int ntiles = (int)(last_key / kKeys) + 1;
    const float *kb = static_cast<const float *>(p.k) + (int64_t)b * p.k_bs + g * D;
    const float *vb = static_cast<const float *>(p.v) + (int64_t)b * p.v_bs + g * D;

    for (int kt = 0; kt < ntiles; ++kt) {
        __syncthreads();
        for (int idx = threadIdx.x; idx < kKeys * D / 4; idx += kRows) {
            const int key = idx / (D / 4), seg = idx % (D / 4);
            const int64_t j = (int64_t)kt * kKeys + key;
            float4 kv = make_float4(0, 0, 0, 0), vv = make_float4(0, 0, 0, 0);
            if (j < tk) {
                kv = *reinterpret_cast<const float4 *>(kb + j * p.k_rs + 4 * seg);
                vv = *reinterpret_cast<const float4 *>(vb + j * p.v_rs + 4 * seg);
            }
            ks[idx] = kv;
            vs[idx] = vv;
        }
        __syncthreads();

        float s[kKeys];
        float mx = -INFINITY;
#pragma unroll
        for (int jj = 0; jj < kKeys; ++jj) {
            float acc = 0.f;
#pragma unroll
            for (int e = 0; e < D / 4; ++e) {
                const float4 kk = ks[jj * (D / 4) + e];
                acc = fmaf(q[4 * e], kk.x, acc);
                acc = fmaf(q[4 * e + 1], kk.y, acc);
                acc = fmaf(q[4 * e + 2], kk.z, acc);
                acc = fmaf(q[4 * e + 3], kk.w, acc);
            }
            const int64_t j = (int64_t)kt * kKeys + jj;
            const bool vis = j < tk && (!CAUSAL || j <= r + qoff);
            s[jj] = vis ? acc * C : -INFINITY;
            mx = fmaxf(mx, s[jj]);
        }
        const float m_new = fmaxf(m, mx);
        const float alpha = m_new == -INFINITY ? 1.f : fast_exp2(m - m_new);
        float psum = 0.f;
#pragma unroll
        for (int jj = 0; jj < kKeys; ++jj) {
            s[jj] = m_new == -INFINITY ? 0.f : fast_exp2(s[jj] - m_new);
            psum += s[jj];
        }
        l = l * alpha + psum;
        m = m_new;
#pragma unroll
        for (int e = 0; e < D; ++e) o[e] *= alpha;
#pragma unroll
        for (int jj = 0; jj < kKeys; ++jj) {
#pragma unroll
            for (int e = 0; e < D / 4; ++e) {
                const float4 vv = vs[jj * (D / 4) + e];
                o[4 * e] = fmaf(s[jj], vv.x, o[4 * e]);
                o[4 * e + 1] = fmaf(s[jj], vv.y, o[4 * e + 1]);
                o[4 * e + 2] = fmaf(s[jj], vv.z, o[4 * e + 2]);
                o[4 * e + 3] = fmaf(s[jj], vv.w, o[4 * e + 3]);
            }
        }
    }
    if (row_ok) {
        const float inv = bad_seq ? __builtin_nanf("") : (l > 0.f ? 1.0f / l : 0.f);
        float *ob = static_cast<float *>(p.out) + b * p.o_bs + r * p.o_rs + h * D;
#pragma unroll
        for (int e = 0; e < D; e += 4)
            *reinterpret_cast<float4 *>(ob + e) =
                make_float4(o[e] * inv, o[e + 1] * inv, o[e + 2] * inv, o[e + 3] * inv);
    }
}

template <int D, bool CAUSAL>
void launch_f32_d(const PrefillLaunch &a, hipStream_t stream) {
    const dim3 grid((unsigned)((a.seq + kRows - 1) / kRows), (unsigned)a.hq, (unsigned)a.batch);
    if (a.prep_q)
        hipLaunchKernelGGL((prefill_f32_kernel<D, CAUSAL, true>), grid, dim3(kRows), 0, stream, a);
    else
        hipLaunchKernelGGL((prefill_f32_kernel<D, CAUSAL, false>), grid, dim3(kRows), 0, stream, a);
}

}  // namespace

hipError_t launch_prefill_f32(const PrefillLaunch &a, hipStream_t stream) {
    if (a.d == 64) {
        if (a.causal) launch_f32_d<64, true>(a, stream); else launch_f32_d<64, false>(a, stream);
    } else {
        if (a.causal) launch_f32_d<128, true>(a, stream); else launch_f32_d<128, false>(a, stream);
    }
    return hipGetLastError();
}

}  // namespace attn
