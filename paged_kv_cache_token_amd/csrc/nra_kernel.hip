// Fused Q/K RMSNorm + RoPE + (FP8) quantisation + paged KV append for gfx950.
//
// Operation: FlashInfer PR "fused QK RMSNorm + NeoX RoPE + FP8 E4M3 quantize +
// NHD paged-KV append" (Contract), TensorRT-LLM PR "Fuse Qwen3.5 gated QKV
// preprocessing" (Phase 2: Gemma norm + RoPE folded into the KV-append
// pass, strided rows), SGLang PR "fused Q/K RMSNorm + RoPE with
// cos_sin_cache" (fp32 table, int64 positions).
//
// Mapping onto CDNA4 (one launch per call, 256-thread workgroups = 4 wave64):
//  * A head row of D bf16 elements is owned by G = D/16 lanes (8 for D=128,
//    16 for D=256).  Lane l of the group loads two 16-byte vectors: elements
//    [8l, 8l+8) and [D/2 + 8l, D/2 + 8l + 8).  Every NeoX pair (i, i + D/2)
//    and every interleaved pair (2i, 2i+1) then sits in one lane's registers:
//    RoPE needs no LDS and no lane exchange.  A wave covers 64/G head rows.
//  * The sum of squares and the FP8 amax are reduced over the G lanes of the
//    row only (DPP within the lane group), never across rows or tokens.
//  * The cos/sin values of a token are loaded straight into the registers of
//    the lanes that use them (each lane needs exactly the 16 values of its
//    own dims) and reused for every head row of that token the wave
//    processes; no LDS staging is needed for them.
//  * Work is cut into tiles.  A token tile holds `tokens_per_tile`
//    consecutive tokens; its (token, chunk of 64/G head rows) items are
//    split into 4 contiguous runs, one per wave, so a wave usually keeps one
//    token's cos/sin for several chunks.  A request tile clears the tails of
//    its requests' last pages and writes their flags.  The grid is
//    persistent: workgroup w takes tiles w, w + gridDim.x, ...
//  * All-or-nothing validation without a host sync or a second kernel:
//    every workgroup stages q_indptr / seq_lens in LDS, checks every request
//    and every page id the call will write (the pages are enumerated
//    through a block-wide prefix sum so each thread checks ~1 page), and
//    reduces the verdict with a barrier.  Every workgroup reads the same
//    metadata, so all reach the same verdict.  An invalid call leaves every
//    token tile idle and makes the request tiles write -1 flags.
#include <type_traits>

#include "qkprep_device.h"
#include "qkprep_internal.h"

namespace qkprep {

namespace {

// first index i in [0, n) with a[i] > key (a non-decreasing), n if none
__device__ __forceinline__ int lds_upper_bound(const int* a, int n, int key) {
    int lo = 0, hi = n;
    while (lo < hi) {
        int mid = (lo + hi) >> 1;
        if (a[mid] <= key) lo = mid + 1; else hi = mid;
    }
    return lo;
}

struct ReqPages {
    int first;   // first logical page this call writes for the request
    int count;   // number of pages (0 if none or if the request is invalid)
    int bad;
};

// Local checks of request b (contract validation + page-count bound) and the
// range of logical pages the call writes for it.
__device__ __forceinline__ ReqPages request_pages(const NraDevArgs& a, const int* s_indptr,
                                                  const int* s_seqlen, int b) {
    ReqPages r{0, 0, 0};
    const int beg = s_indptr[b], end = s_indptr[b + 1];
    const int ql = end - beg;
    const int sl = s_seqlen[b];
    if (ql < 0 || sl < ql || (int64_t)sl > (int64_t)a.maxp * a.page_size ||
        (a.q_scale_padded && ql > a.max_seqlen)) {
        r.bad = 1;
        return r;
    }
    int lo_row = sl - ql;
    if (a.zero_tail && ql == 0 && sl > 0) lo_row = sl - 1;
    if (sl > lo_row) {
        r.first = lo_row / a.page_size;
        r.count = (sl - 1) / a.page_size - r.first + 1;
    }
    return r;
}

// Block-wide verdict over the whole call (see file comment).  Fills
// s_indptr[0..B], s_seqlen[0..B) and s_pre[0..B] (exclusive prefix of the
// per-request page counts).  Returns non-zero when the call is invalid.
__device__ int validate_call(const NraDevArgs& a, int* s_indptr, int* s_seqlen, int* s_pre,
                             int* s_wave) {
    const int tid = threadIdx.x;
    const int B = a.B;
    int bad = 0;
    for (int i = tid; i <= B; i += kBlockThreads) s_indptr[i] = a.q_indptr[i];
    for (int i = tid; i < B; i += kBlockThreads) s_seqlen[i] = a.seq_lens[i];
    __syncthreads();
    if (tid == 0 && (s_indptr[0] != 0 || s_indptr[B] != a.T)) bad = 1;

    // per-thread run of consecutive requests -> page counts -> block scan
    const int per = (B + kBlockThreads - 1) / kBlockThreads;
    const int lo = min(B, tid * per), hi = min(B, lo + per);
    int sum = 0;
    for (int b = lo; b < hi; ++b) {
        ReqPages rp = request_pages(a, s_indptr, s_seqlen, b);
        bad |= rp.bad;
        sum += rp.count;
    }
    const int lane = tid & 63, wave = tid >> 6;
    int incl = sum;
#pragma unroll
    for (int off = 1; off < 64; off <<= 1) {
        int up = __shfl_up(incl, off, 64);
        if (lane >= off) incl += up;
    }
    if (lane == 63) s_wave[wave] = incl;
    __syncthreads();
    int base = 0;
    for (int w = 0; w < wave; ++w) base += s_wave[w];
    int run = base + incl - sum;
    for (int b = lo; b < hi; ++b) {
        s_pre[b] = run;
        run += request_pages(a, s_indptr, s_seqlen, b).count;
    }
    if (tid == kBlockThreads - 1) s_pre[B] = base + incl;
    __syncthreads();

    // every page id the call writes must lie in the pool
    const int total = s_pre[B];
    for (int k = tid; k < total; k += kBlockThreads) {
        const int b = lds_upper_bound(s_pre, B + 1, k) - 1;
        const ReqPages rp = request_pages(a, s_indptr, s_seqlen, b);
        const int pidx = rp.first + (k - s_pre[b]);
        const int p = a.page_table[(int64_t)b * a.maxp + pidx];
        if (p < 0 || p >= a.num_pages) bad = 1;
    }
    return __syncthreads_or(bad);
}

template <int D, int QMODE, bool KVFP8>
__global__ __launch_bounds__(kBlockThreads) void nra_kernel(const NraDevArgs a) {
    constexpr int G = D / 16;        // lanes per head row
    constexpr int RPW = 64 / G;      // head rows per wave
    constexpr int HALF = D / 2;

    extern __shared__ int s_dyn[];   // q_indptr [B+1] | seq_lens [B] | page prefix [B+1]
    __shared__ int s_wave[4];
    __shared__ int s_pos[kMaxTokensPerTile];
    __shared__ int64_t s_koff[kMaxTokensPerTile];
    __shared__ int64_t s_voff[kMaxTokensPerTile];
    __shared__ int64_t s_qsoff[kMaxTokensPerTile];

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = tid >> 6;
    const int grp = lane / G;        // head-row slot of this lane in the wave
    const int gl = lane % G;         // lane inside the head row

    int* s_indptr = s_dyn;
    int* s_seqlen = s_dyn + (a.B + 1);
    int* s_pre = s_dyn + (2 * a.B + 1);

    int bad = 0;
    if (a.paged) bad = validate_call(a, s_indptr, s_seqlen, s_pre, s_wave);

    // per-lane norm weights for the lane's 16 dims
    float wq[16], wk[16];
    if (a.norm != 0) {
        const float add = (a.norm == 2) ? 1.0f : 0.0f;
#pragma unroll
        for (int h = 0; h < 2; ++h) {
            const int off = h * HALF + 8 * gl;
            float4 q0 = ldf4(a.q_w + off), q1 = ldf4(a.q_w + off + 4);
            float4 k0 = ldf4(a.k_w + off), k1 = ldf4(a.k_w + off + 4);
            wq[8 * h + 0] = q0.x + add; wq[8 * h + 1] = q0.y + add;
            wq[8 * h + 2] = q0.z + add; wq[8 * h + 3] = q0.w + add;
            wq[8 * h + 4] = q1.x + add; wq[8 * h + 5] = q1.y + add;
            wq[8 * h + 6] = q1.z + add; wq[8 * h + 7] = q1.w + add;
            wk[8 * h + 0] = k0.x + add; wk[8 * h + 1] = k0.y + add;
            wk[8 * h + 2] = k0.z + add; wk[8 * h + 3] = k0.w + add;
            wk[8 * h + 4] = k1.x + add; wk[8 * h + 5] = k1.y + add;
            wk[8 * h + 6] = k1.z + add; wk[8 * h + 7] = k1.w + add;
        }
    } else {
#pragma unroll
        for (int i = 0; i < 16; ++i) { wq[i] = 1.0f; wk[i] = 1.0f; }
    }
    const float inv_k = KVFP8 ? 1.0f / *a.k_scale : 1.0f;
    const float inv_v = KVFP8 ? 1.0f / *a.v_scale : 1.0f;
    const float q_static = (QMODE == 2) ? *a.q_scale_inv : 1.0f;
    const float inv_D = 1.0f / (float)D;

    typedef typename std::conditional<KVFP8, uint8_t, uint16_t>::type kv_t;
    kv_t* kc = reinterpret_cast<kv_t*>(a.k_cache);
    kv_t* vc = reinterpret_cast<kv_t*>(a.v_cache);
    const int64_t row_elems = (int64_t)a.Hkv * D;
    const int TPB = a.tokens_per_tile;
    const int CPT = a.chunks_per_token;
    const int n_tiles = a.n_req_tiles + a.n_token_tiles;

    for (int tile = blockIdx.x; tile < n_tiles; tile += gridDim.x) {
        if (tile < a.n_req_tiles) {
            // ---------------- request tile: flags and tail clear ----------------
            for (int bi = 0; bi < a.reqs_per_tile; ++bi) {
                const int b = tile * a.reqs_per_tile + bi;
                if (b >= a.B) break;
                for (int h = tid; h < a.Hkv; h += kBlockThreads)
                    a.flags[(int64_t)b * a.Hkv + h] = bad ? -1 : 0;
                if (bad || !a.zero_tail) continue;
                const int sl = s_seqlen[b];
                if (sl <= 0) continue;
                const int last = (sl - 1) % a.page_size;
                const int64_t page = a.page_table[(int64_t)b * a.maxp + (sl - 1) / a.page_size];
                const int64_t nvec = (int64_t)(a.page_size - 1 - last) * row_elems * sizeof(kv_t) / 16;
                char* kb = reinterpret_cast<char*>(kc + page * a.k_page_stride + (last + 1) * row_elems);
                char* vb = reinterpret_cast<char*>(vc + page * a.v_page_stride + (last + 1) * row_elems);
                const uint4 z = make_uint4(0, 0, 0, 0);
                for (int64_t i = tid; i < nvec; i += kBlockThreads) {
                    st16(kb + 16 * i, z);
                    st16(vb + 16 * i, z);
                }
            }
            continue;
        }
        if (bad) continue;

        // ---------------- token tile ----------------
        const int t0 = (tile - a.n_req_tiles) * TPB;
        if (tid < TPB) {
            const int t = t0 + tid;
            int pos = -1;
            int64_t koff = -1, voff = -1, qsoff = 0;
            if (t < a.T) {
                const int64_t p64 = a.positions[t];
                if (p64 >= 0 && p64 < a.cs_rows) pos = (int)p64;
                if (a.paged) {
                    const int b = lds_upper_bound(s_indptr, a.B + 1, t) - 1;
                    const int beg = s_indptr[b];
                    const int ql = s_indptr[b + 1] - beg;
                    const int j = t - beg;
                    const int L = s_seqlen[b] - ql + j;
                    const int64_t page = a.page_table[(int64_t)b * a.maxp + L / a.page_size];
                    const int64_t row = L % a.page_size;
                    koff = page * a.k_page_stride + row * row_elems;
                    voff = page * a.v_page_stride + row * row_elems;
                    qsoff = a.q_scale_padded ? (int64_t)b * a.Hq * a.q_scale_P + j : (int64_t)t * a.Hq;
                } else {
                    const int64_t slot = a.slot_mapping[t];
                    if (slot >= 0 && slot < (int64_t)a.num_pages * a.page_size) {
                        const int64_t page = slot / a.page_size, row = slot % a.page_size;
                        koff = page * a.k_page_stride + row * row_elems;
                        voff = page * a.v_page_stride + row * row_elems;
                    }
                    qsoff = (int64_t)t * a.Hq;
                }
            }
            s_pos[tid] = pos;
            s_koff[tid] = koff;
            s_voff[tid] = voff;
            s_qsoff[tid] = qsoff;
        }
        __syncthreads();

        const int n_items = TPB * CPT;
        const int ipw = (n_items + 3) >> 2;
        const int it_lo = wave * ipw;
        const int it_hi = min(n_items, it_lo + ipw);
        const int qs_hstride = a.q_scale_padded ? (int)a.q_scale_P : 1;
        int cur_ti = -1;
        float c[8], s[8];
        for (int it = it_lo; it < it_hi; ++it) {
            const int ti = it / CPT;
            const int chunk = it - ti * CPT;
            const int t = t0 + ti;
            if (t >= a.T) break;
            const int pos = s_pos[ti];
            if (pos < 0) continue;
            if (ti != cur_ti) {
                cur_ti = ti;
                const float* cs = a.cos_sin + (int64_t)pos * D;
                if (a.rope == 0) {
                    // NeoX: pair k of the lane has angle 8*gl + k
                    float4 c0 = ldf4(cs + 8 * gl), c1 = ldf4(cs + 8 * gl + 4);
                    float4 s0 = ldf4(cs + HALF + 8 * gl), s1 = ldf4(cs + HALF + 8 * gl + 4);
                    c[0] = c0.x; c[1] = c0.y; c[2] = c0.z; c[3] = c0.w;
                    c[4] = c1.x; c[5] = c1.y; c[6] = c1.z; c[7] = c1.w;
                    s[0] = s0.x; s[1] = s0.y; s[2] = s0.z; s[3] = s0.w;
                    s[4] = s1.x; s[5] = s1.y; s[6] = s1.z; s[7] = s1.w;
                } else {
                    // interleaved: first vector holds angles 4*gl .. 4*gl+3,
                    // second vector angles D/4 + 4*gl .. D/4 + 4*gl + 3
                    float4 c0 = ldf4(cs + 4 * gl), c1 = ldf4(cs + D / 4 + 4 * gl);
                    float4 s0 = ldf4(cs + HALF + 4 * gl), s1 = ldf4(cs + HALF + D / 4 + 4 * gl);
                    c[0] = c0.x; c[1] = c0.y; c[2] = c0.z; c[3] = c0.w;
                    c[4] = c1.x; c[5] = c1.y; c[6] = c1.z; c[7] = c1.w;
                    s[0] = s0.x; s[1] = s0.y; s[2] = s0.z; s[3] = s0.w;
                    s[4] = s1.x; s[5] = s1.y; s[6] = s1.z; s[7] = s1.w;
                }
            }
            const int r = chunk * RPW + grp;          // head row of this lane group
            if (r >= a.R) continue;                   // idle group (lane-group uniform)
            const uint16_t* src = a.qkv + (int64_t)t * a.qkv_stride + (int64_t)r * D + 8 * gl;
            const uint4 v0 = ld16(src);
            const uint4 v1 = ld16(src + HALF);
            if (r >= a.Hq + a.Hkv) {
                // V head: raw copy (bf16 cache) or x / v_scale (FP8 cache)
                const int64_t voff = s_voff[ti];
                if (voff < 0) continue;
                kv_t* dst = vc + voff + (int64_t)(r - a.Hq - a.Hkv) * D + 8 * gl;
                if constexpr (KVFP8) {
                    float x[16];
                    unpack8(v0, x);
                    unpack8(v1, x + 8);
                    st8(dst, pack8_fp8(x, inv_v));
                    st8(dst + HALF, pack8_fp8(x + 8, inv_v));
                } else {
                    st16(dst, v0);
                    st16(dst + HALF, v1);
                }
                continue;
            }
            const bool is_q = r < a.Hq;
            float x[16];
            unpack8(v0, x);
            unpack8(v1, x + 8);
            if (a.norm != 0) {
                float ss = 0.0f;
#pragma unroll
                for (int k = 0; k < 16; ++k) ss = fmaf(x[k], x[k], ss);
                ss = group_sum<G>(ss);
                const float inv = rsqrtf(fmaf(ss, inv_D, a.eps));
#pragma unroll
                for (int k = 0; k < 16; ++k) x[k] = x[k] * inv * (is_q ? wq[k] : wk[k]);
            }
            if (a.rope == 0) {
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
            if (is_q) {
                const int h = r;
                if constexpr (QMODE == 0) {
                    uint16_t* dst = reinterpret_cast<uint16_t*>(a.q_out) + (int64_t)t * a.q_out_stride +
                                    (int64_t)h * D + 8 * gl;
                    st16(dst, pack8_bf16(x));
                    st16(dst + HALF, pack8_bf16(x + 8));
                } else {
                    uint8_t* dst = reinterpret_cast<uint8_t*>(a.q_out) + (int64_t)t * a.q_out_stride +
                                   (int64_t)h * D + 8 * gl;
                    float mul = q_static;
                    if constexpr (QMODE == 1) {
                        float amax = 0.0f;
#pragma unroll
                        for (int k = 0; k < 16; ++k) amax = __builtin_fmaxf(amax, __builtin_fabsf(x[k]));
                        amax = group_max<G>(amax);
                        const float sc = __builtin_fmaxf(amax, 1e-6f) / a.upper_max;
                        mul = 1.0f / sc;
                        if (gl == 0) a.q_scale[s_qsoff[ti] + (int64_t)h * qs_hstride] = sc;
                    }
                    st8(dst, pack8_fp8(x, mul));
                    st8(dst + HALF, pack8_fp8(x + 8, mul));
                }
            } else {
                const int kh = r - a.Hq;
                const int64_t koff = s_koff[ti];
                if (koff >= 0) {
                    kv_t* dst = kc + koff + (int64_t)kh * D + 8 * gl;
                    if constexpr (KVFP8) {
                        st8(dst, pack8_fp8(x, inv_k));
                        st8(dst + HALF, pack8_fp8(x + 8, inv_k));
                    } else {
                        st16(dst, pack8_bf16(x));
                        st16(dst + HALF, pack8_bf16(x + 8));
                    }
                }
                if (a.k_out) {
                    uint16_t* ko = a.k_out + (int64_t)t * a.k_out_stride + (int64_t)kh * D + 8 * gl;
                    st16(ko, pack8_bf16(x));
                    st16(ko + HALF, pack8_bf16(x + 8));
                }
            }
        }
        __syncthreads();   // the next tile rewrites the per-token LDS arrays
    }
}

template <int D, int QMODE, bool KVFP8>
hipError_t launch_t(const NraDevArgs& a, hipStream_t stream) {
    const int n_tiles = a.n_req_tiles + a.n_token_tiles;
    const int grid = n_tiles < 8192 ? n_tiles : 8192;
    const size_t lds = a.paged ? (size_t)(3 * a.B + 2) * sizeof(int) : 0;
    hipLaunchKernelGGL((nra_kernel<D, QMODE, KVFP8>), dim3(grid), dim3(kBlockThreads), lds, stream, a);
    return hipGetLastError();
}

}  // namespace

hipError_t launch_norm_rope_append(const NraDevArgs& a, int head_dim, int q_mode, int kv_fp8,
                                   hipStream_t stream) {
#define QKPREP_NRA_CASE(DD, QM, KF) \
    if (head_dim == DD && q_mode == QM && (kv_fp8 != 0) == KF) return launch_t<DD, QM, KF>(a, stream);
    QKPREP_NRA_CASE(128, 0, false) QKPREP_NRA_CASE(128, 0, true)
    QKPREP_NRA_CASE(128, 1, false) QKPREP_NRA_CASE(128, 1, true)
    QKPREP_NRA_CASE(128, 2, false) QKPREP_NRA_CASE(128, 2, true)
    QKPREP_NRA_CASE(256, 0, false) QKPREP_NRA_CASE(256, 0, true)
    QKPREP_NRA_CASE(256, 1, false) QKPREP_NRA_CASE(256, 1, true)
    QKPREP_NRA_CASE(256, 2, false) QKPREP_NRA_CASE(256, 2, true)
#undef QKPREP_NRA_CASE
    return hipErrorInvalidValue;
}

}  // namespace qkprep
