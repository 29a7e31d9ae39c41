// MLA latent-cache append for gfx950: RoPE on the rope slice of every q head
// (in place) and the [kv_c | RoPE(k_pe)] concat into the latent cache.
//
// Operation: vLLM issue "ROPE + KV-Cache-Write + pre-attn prepare-ops fusion"
// (concat_and_cache_mla / concat_cache_mla_rope; DeepSeek-R1: 128 heads, 64
// rope dims, 128 nope dims, latent 512, RoPE on interleaved pairs).
//
// Mapping onto CDNA4 (256-thread workgroups = 4 wave64):
//  * The 64-element rope slice of one q head (128 bytes) is owned by 4 lanes.
//    Lane l loads elements [8l, 8l+8) and [32 + 8l, 32 + 8l + 8); NeoX pairs
//    (i, i + 32) and interleaved pairs (2i, 2i+1) are then both lane-local.
//    A wave covers 16 heads; the nope part of q is never touched.
//  * Per token: ceil(H / 16) q chunks plus one latent chunk in which the 64
//    lanes convert 8 latent elements each (512 per pass) and lanes 0..3
//    rotate and convert k_pe.  cos/sin live in the registers of the lanes
//    that use them.
//  * Tiles of `tokens_per_tile` tokens, items split into 4 contiguous runs,
//    persistent grid.
#include <type_traits>

#include "qkprep_device.h"
#include "qkprep_internal.h"

namespace qkprep {

namespace {

constexpr int kRope = 64;                 // rope dims handled by this kernel
constexpr int kHalf = kRope / 2;
constexpr int kLanesPerHead = 4;
constexpr int kHeadsPerWave = 64 / kLanesPerHead;

__device__ __forceinline__ void rope16(float* x, const float* c, const float* s, int style) {
    if (style == 0) {
#pragma unroll
        for (int k = 0; k < 8; ++k) {
            const float xa = x[k], xb = x[8 + k];
            x[k] = xa * c[k] - xb * s[k];
            x[8 + k] = xb * c[k] + xa * s[k];
        }
    } else {
#pragma unroll
        for (int m = 0; m < 8; ++m) {
            const int i0 = (m < 4) ? 2 * m : 8 + 2 * (m - 4);
            const float xa = x[i0], xb = x[i0 + 1];
            x[i0] = xa * c[m] - xb * s[m];
            x[i0 + 1] = xb * c[m] + xa * s[m];
        }
    }
}

template <bool KVFP8>
__global__ __launch_bounds__(kBlockThreads) void mla_kernel(const MlaDevArgs a) {
    __shared__ int s_pos[kMaxTokensPerTile];
    __shared__ int64_t s_row[kMaxTokensPerTile];   // element offset of the cache row, -1 = skip

    preload_kernargs(a);
    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = tid >> 6;
    const int grp = lane / kLanesPerHead;
    const int gl = lane % kLanesPerHead;
    const int K = a.kv_lora_rank;
    const int row_len = K + kRope;
    const int n_qchunks = a.chunks_per_token - 1;
    const int TPB = a.tokens_per_tile;
    const float inv_scale = KVFP8 ? 1.0f / *a.kv_scale : 1.0f;

    typedef typename std::conditional<KVFP8, uint8_t, uint16_t>::type kv_t;
    kv_t* cache = reinterpret_cast<kv_t*>(a.kv_cache);

    for (int tile = blockIdx.x; tile < a.n_tiles; tile += a.grid) {
        const int t0 = tile * TPB;
        if (tid < TPB) {
            const int t = t0 + tid;
            int pos = -1;
            int64_t row = -1;
            if (t < a.T) {
                const int64_t p64 = a.positions[t];
                if (p64 >= 0 && p64 < a.cs_rows) pos = (int)p64;
                const int64_t slot = a.slot_mapping[t];
                if (slot >= 0 && slot < a.capacity)
                    row = (slot / a.block_size) * a.block_stride + (slot % a.block_size) * (int64_t)row_len;
            }
            s_pos[tid] = pos;
            s_row[tid] = row;
        }
        __syncthreads();

        const int n_items = TPB * a.chunks_per_token;
        const int ipw = (n_items + 3) >> 2;
        const int it_lo = wave * ipw;
        const int it_hi = min(n_items, it_lo + ipw);
        int cur_ti = -1;
        float c[8], s[8];
        for (int it = it_lo; it < it_hi; ++it) {
            const int ti = it / a.chunks_per_token;
            const int chunk = it - ti * a.chunks_per_token;
            const int t = t0 + ti;
            if (t >= a.T) break;
            const int pos = s_pos[ti];
            if (pos < 0) continue;
            if (ti != cur_ti) {
                cur_ti = ti;
                const float* cs = a.cos_sin + (int64_t)pos * kRope;
                float4 c0, c1, s0, s1;
                if (a.rope == 0) {
                    c0 = ldf4(cs + 8 * gl); c1 = ldf4(cs + 8 * gl + 4);
                    s0 = ldf4(cs + kHalf + 8 * gl); s1 = ldf4(cs + kHalf + 8 * gl + 4);
                } else {
                    c0 = ldf4(cs + 4 * gl); c1 = ldf4(cs + kRope / 4 + 4 * gl);
                    s0 = ldf4(cs + kHalf + 4 * gl); s1 = ldf4(cs + kHalf + kRope / 4 + 4 * gl);
                }
                c[0] = c0.x; c[1] = c0.y; c[2] = c0.z; c[3] = c0.w;
                c[4] = c1.x; c[5] = c1.y; c[6] = c1.z; c[7] = c1.w;
                s[0] = s0.x; s[1] = s0.y; s[2] = s0.z; s[3] = s0.w;
                s[4] = s1.x; s[5] = s1.y; s[6] = s1.z; s[7] = s1.w;
            }
            if (chunk < n_qchunks) {
                // ---- q rope slice of head h, in place ----
                const int h = chunk * kHeadsPerWave + grp;
                if (h >= a.H) continue;
                uint16_t* p = a.q + (int64_t)t * a.q_token_stride + (int64_t)h * a.q_head_stride +
                              a.nope_dim + 8 * gl;
                float x[16];
                unpack8(ld16(p), x);
                unpack8(ld16(p + kHalf), x + 8);
                rope16(x, c, s, a.rope);
                st16(p, pack8_bf16(x));
                st16(p + kHalf, pack8_bf16(x + 8));
                continue;
            }
            // ---- latent chunk: [kv_c | RoPE(k_pe)] -> cache row ----
            const int64_t row = s_row[ti];
            if (row < 0) continue;
            kv_t* dst = cache + row;
            const uint16_t* kc = a.kv_c + (int64_t)t * a.kv_c_stride;
            for (int e = 8 * lane; e < K; e += 512) {
                const uint4 v = ld16(kc + e);
                if constexpr (KVFP8) {
                    float x[8];
                    unpack8(v, x);
                    st8(dst + e, pack8_fp8(x, inv_scale));
                } else {
                    st16(dst + e, v);
                }
            }
            if (lane < kLanesPerHead) {
                const uint16_t* kp = a.k_pe + (int64_t)t * a.k_pe_stride + 8 * gl;
                float x[16];
                unpack8(ld16(kp), x);
                unpack8(ld16(kp + kHalf), x + 8);
                rope16(x, c, s, a.rope);
                if constexpr (KVFP8) {
                    store_fp8_row(reinterpret_cast<uint8_t*>(dst + K), gl, kHalf, pack8_fp8(x, inv_scale),
                                  pack8_fp8(x + 8, inv_scale));
                } else {
                    st16(dst + K + 8 * gl, pack8_bf16(x));
                    st16(dst + K + kHalf + 8 * gl, pack8_bf16(x + 8));
                }
            }
        }
        __syncthreads();
    }
}

template <bool KVFP8>
hipError_t launch_t(const MlaDevArgs& a, hipStream_t stream) {
    MlaDevArgs la = a;
    la.grid = a.n_tiles < 8192 ? a.n_tiles : 8192;
    hipLaunchKernelGGL((mla_kernel<KVFP8>), dim3(la.grid), dim3(kBlockThreads), 0, stream, la);
    return hipGetLastError();
}

}  // namespace

hipError_t launch_mla_concat_rope(const MlaDevArgs& a, int kv_fp8, hipStream_t stream) {
    return kv_fp8 ? launch_t<true>(a, stream) : launch_t<false>(a, stream);
}

}  // namespace qkprep
