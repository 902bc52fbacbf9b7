// kernels.h -- host-side launchers of the HIP kernels (internal to libattn).
//
// The C ABI layer (attn_api.cpp) validates every argument and then calls these.
// They only configure and enqueue launches; each returns the hipError_t of the
// enqueue.  Strides are in elements.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace attn {

// HeadPrep of the tokens [0, seq) of `batch` sequences, for q and/or k.  src and dst
// may be the same buffer (in place).  Token t uses table row pos0 + t.
struct PrepLaunch {
    const void *q_src; void *q_dst; int64_t q_src_rs, q_dst_rs; int64_t hq;
    const void *k_src; void *k_dst; int64_t k_src_rs, k_dst_rs; int64_t hkv;
    int64_t batch, seq, d, pos0;
    const float *qw, *kw, *cos, *sin;
    int64_t half;
    float eps;
    bool bf16;
};
hipError_t launch_prep(const PrepLaunch &a, hipStream_t stream);

// Attention of whole sequences.  When q_prepped is false and prep tables are given,
// q's HeadPrep is applied as the q rows are read (k must already be prepped).
struct PrefillLaunch {
    const void *q; const void *k; const void *v; void *out;
    int64_t q_rs, k_rs, v_rs, o_rs;
    int64_t batch, seq, hq, hkv, d, pos0;
    bool prep_q;                 // apply HeadPrep to q in the prologue
    const float *qw, *cos, *sin;
    int64_t half;
    float eps;
    bool causal;
    float scale;
    bool bf16;
};
hipError_t launch_prefill(const PrefillLaunch &a, hipStream_t stream);
// true if the fused q prologue of the chosen kernel can turn pairs `half` apart.
bool prefill_fuses_half(int64_t d, int64_t half, bool bf16);

struct DecodeLaunch {
    const void *q; const void *k; const void *v; void *out;
    int64_t batch, hq, hkv, d, capacity, max_len;
    const int32_t *lens, *pos;
    bool prep_q;
    const float *qw, *cos, *sin;
    int64_t half, table_rows;
    float eps;
    float scale;
    int64_t splits;
    float *work;                 // [splits][batch][hq] x (d + 2) f32 partials
    bool bf16;
};
hipError_t launch_decode(const DecodeLaunch &a, hipStream_t stream);

// Geometry of the decode split kernel, shared with the ABI layer's size queries.
int64_t decode_heads_per_block(int64_t hq, int64_t hkv);
int64_t decode_default_splits(int64_t batch, int64_t hq, int64_t hkv, int64_t max_len);
size_t decode_workspace_bytes(int64_t batch, int64_t hq, int64_t d, int64_t splits);

}  // namespace attn
