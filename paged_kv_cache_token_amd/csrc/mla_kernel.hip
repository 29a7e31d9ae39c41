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
//    A wave covers 16 heads (a "q chunk"); the nope part of q is never read.
//  * Per token: ceil(H / 16) q chunks plus one latent chunk.  In the latent
//    chunk each of the 64 lanes loads 8 latent elements (512 per pass) and
//    lanes 0..7 load the 64 k_pe elements; lanes 0..3 take the second half
//    of k_pe from lanes 4..7, rotate it and convert it.
//  * Every chunk issues exactly two 16-byte loads per lane, so the loads of
//    the next two chunks are issued before the stores of the current ones
//    with exact wait counts (double buffering).
//  * Every workgroup owns a balanced, contiguous range of about 8 (token,
//    chunk) items (more workgroups than stay resident); tiles of up to 16
//    tokens stage their cos/sin rows (64 floats), positions and cache-row
//    offsets in LDS.
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

// the 16 cos/sin values lane gl of a head needs, from the LDS row of its token
__device__ __forceinline__ void lane_cos_sin(const float* row, int gl, int style, float* c, float* s) {
    float4 c0, c1, s0, s1;
    if (style == 0) {
        c0 = *reinterpret_cast<const float4*>(row + 8 * gl);
        c1 = *reinterpret_cast<const float4*>(row + 8 * gl + 4);
        s0 = *reinterpret_cast<const float4*>(row + kHalf + 8 * gl);
        s1 = *reinterpret_cast<const float4*>(row + kHalf + 8 * gl + 4);
    } else {
        c0 = *reinterpret_cast<const float4*>(row + 4 * gl);
        c1 = *reinterpret_cast<const float4*>(row + kRope / 4 + 4 * gl);
        s0 = *reinterpret_cast<const float4*>(row + kHalf + 4 * gl);
        s1 = *reinterpret_cast<const float4*>(row + kHalf + kRope / 4 + 4 * gl);
    }
    c[0] = c0.x; c[1] = c0.y; c[2] = c0.z; c[3] = c0.w;
    c[4] = c1.x; c[5] = c1.y; c[6] = c1.z; c[7] = c1.w;
    s[0] = s0.x; s[1] = s0.y; s[2] = s0.z; s[3] = s0.w;
    s[4] = s1.x; s[5] = s1.y; s[6] = s1.z; s[7] = s1.w;
}

struct MlaCursor {
    int t, c, left;
    __device__ __forceinline__ void advance(int cpt) {
        const bool wrap = c + 1 == cpt;
        c = wrap ? 0 : c + 1;
        t += wrap ? 1 : 0;
        --left;
    }
};

// element offset of cache slot `slot` (0 <= slot < capacity)
__device__ __forceinline__ int64_t cache_row(const MlaDevArgs& a, int64_t slot, int row_len) {
    int64_t blk, in;
    if (a.capacity <= INT32_MAX) {
        blk = fdiv31((int)slot, a.bs_div);
        in = slot - blk * a.block_size;
    } else {
        blk = slot / a.block_size;
        in = slot % a.block_size;
    }
    return blk * a.block_stride + in * (int64_t)row_len;
}

// read by the load slots past a wave's run; never written
__device__ __align__(16) const uint16_t g_mla_zero[8] = {};

template <bool KVFP8, bool NT>
__global__ __launch_bounds__(kBlockThreads) void mla_kernel(const MlaDevArgs a) {
    constexpr int U = kBatch;
    typedef typename std::conditional<KVFP8, uint8_t, uint16_t>::type kv_t;
    __shared__ __align__(16) float s_cs[kMaxTokensPerTile * kRope];
    __shared__ int s_pos[kMaxTokensPerTile];
    __shared__ int64_t s_row[kMaxTokensPerTile];   // element offset of the cache row, -1 = skip

    preload_kernargs(a);
    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);   // wave-uniform
    const int grp = lane / kLanesPerHead;
    const int gl = lane % kLanesPerHead;
    // element offsets (in the rope slice) of the two whole-line loads and
    // stores of head pair (2p, 2p+1): the even head's lanes read their own
    // first vector and the odd head's lanes the even head's second vector,
    // then the odd head's line the same way
    const bool even_head = (grp & 1) == 0;
    const int q_off0 = even_head ? 8 * gl : 56 - 8 * gl;
    const int q_off1 = even_head ? 24 - 8 * gl : 32 + 8 * gl;
    const int K = a.kv_lora_rank;
    const int row_len = K + kRope;
    const int CPT = a.chunks_per_token;
    const int n_qchunks = CPT - 1;
    const int TPB = a.tokens_per_tile;
    // the scale's load is issued here and its reciprocal taken after the
    // first barrier (taken right away, it would wait for the load on the spot)
    const float kv_scale_v = KVFP8 ? *a.kv_scale : 1.0f;
    float inv_scale = 1.0f;
    kv_t* cache = reinterpret_cast<kv_t*>(a.kv_cache);

    // total * b / grid = items_q * b + items_r * b / grid (items_r * b < grid^2)
    const int blo = a.items_q * (int)blockIdx.x + fdiv31(a.items_r * (int)blockIdx.x, a.grid_div);
    const int bhi = a.items_q * ((int)blockIdx.x + 1) + fdiv31(a.items_r * ((int)blockIdx.x + 1), a.grid_div);
    int sub_lo = blo, sub_hi = blo, t_first = 0, ntok = 0;
    MlaCursor ld{0, 0, 0}, pr{0, 0, 0};
    uint4 bufA[U][2], bufB[U][2];

    // two 16-byte loads per lane per chunk, always issued: rows past the
    // run or heads past H read a 16-byte zero vector that stays in the
    // caches, so that the last batch of a tile does not wait for a memory
    // round trip of its own
    auto load_batch = [&](uint4 (&buf)[U][2]) {
#pragma unroll
        for (int u = 0; u < U; ++u) {
            const bool live = ld.left > 0;
            const int t = live ? ld.t : t_first;
            const uint16_t* p0;
            const uint16_t* p1;
            if (ld.c < n_qchunks) {
                // heads 2p and 2p+1 of the chunk: each load reads one head's
                // whole 128-byte rope slice (mirror_exchange completes them)
                const int ha = ld.c * kHeadsPerWave + (grp & ~1), hb = ha + 1;
                const uint16_t* q = a.q + (int64_t)t * a.q_token_stride + a.nope_dim;
                p0 = live && ha < a.H ? q + (int64_t)ha * a.q_head_stride + q_off0 : g_mla_zero;
                p1 = live && hb < a.H ? q + (int64_t)hb * a.q_head_stride + q_off1 : g_mla_zero;
            } else {
                p0 = live ? a.kv_c + (int64_t)t * a.kv_c_stride + 8 * lane : g_mla_zero;
                p1 = live ? a.k_pe + (int64_t)t * a.k_pe_stride + 8 * (lane & 7) : g_mla_zero;
            }
            buf[u][0] = ld16(p0);
            buf[u][1] = ld16(p1);
            ld.advance(CPT);
        }
    };
    auto start_tile = [&]() {
        t_first = fdiv31(sub_lo, a.cpt_div);
        sub_hi = min(bhi, (t_first + TPB) * CPT);
        ntok = fdiv31(sub_hi - 1, a.cpt_div) - t_first + 1;
        const int n = sub_hi - sub_lo;
        const int w_lo = sub_lo + n * wave / 4;
        const int w_hi = sub_lo + n * (wave + 1) / 4;
        ld.t = fdiv31(w_lo, a.cpt_div);
        ld.c = w_lo - ld.t * CPT;
        ld.left = w_hi - w_lo;
        pr = ld;
    };
    // Tile metadata, in one chain of two rounds with the tile's first q batch
    // issued alongside: every thread loads the position of the cos/sin row
    // piece it stages (thread k: token k / 16, float4 k % 16; ntok <= 16
    // tokens x 16 float4 = 256) and thread i < ntok the token's slot, all
    // unmasked at clamped indices; then the qkv batch; then the cos/sin
    // loads, which need the positions.
    static_assert(kMaxTokensPerTile * (kRope / 4) <= kBlockThreads, "one cos/sin float4 per thread");
    auto stage_tile = [&]() {
        const int ic = min(tid / (kRope / 4), ntok - 1);
        const int c4 = tid % (kRope / 4);
        const int it = min(tid, ntok - 1);
        const int64_t pc = gld(a.positions + t_first + ic);
        const int64_t pt = gld(a.positions + t_first + it);
        const int64_t slot = gld(a.slot_mapping + t_first + it);
        load_batch(bufA);
        const bool pc_ok = pc >= 0 && pc < a.cs_rows;
        const float4 cs = ldf4(a.cos_sin + (pc_ok ? pc : 0) * kRope + 4 * c4);
        if (tid < ntok) {
            s_pos[tid] = (pt >= 0 && pt < a.cs_rows) ? (int)pt : -1;
            s_row[tid] = (slot >= 0 && slot < a.capacity) ? cache_row(a, slot, row_len) : -1;
        }
        if (tid < ntok * (kRope / 4) && pc_ok) *reinterpret_cast<float4*>(s_cs + ic * kRope + 4 * c4) = cs;
    };
    auto run_batch = [&](uint4 (&buf)[U][2]) {
#pragma unroll
        for (int u = 0; u < U; ++u) {
            if (pr.left > 0) {
                const int t = pr.t;
                const int ti = t - t_first;
                const int chunk = pr.c;
                const int pos = s_pos[ti];
                if (chunk < n_qchunks) {
                    // (wave-uniform branch: every lane takes part in the exchanges)
                    mirror_exchange<kDppRowHalfMirror, 0xA, 0x5>(buf[u][0], buf[u][1]);
                    float c[8], s[8], x[16];
                    lane_cos_sin(s_cs + ti * kRope, gl, a.rope, c, s);
                    unpack8(buf[u][0], x);
                    unpack8(buf[u][1], x + 8);
                    rope16(x, c, s, a.rope);
                    uint4 lo = pack8_bf16(x), hi = pack8_bf16(x + 8);
                    // the same exchange turns the lane's own halves into the
                    // whole-line stores at the load addresses
                    mirror_exchange<kDppRowHalfMirror, 0xA, 0x5>(lo, hi);
                    const int ha = chunk * kHeadsPerWave + (grp & ~1), hb = ha + 1;
                    uint16_t* q = a.q + (int64_t)t * a.q_token_stride + a.nope_dim;
                    if (pos >= 0 && ha < a.H) st16p<NT>(q + (int64_t)ha * a.q_head_stride + q_off0, lo);
                    if (pos >= 0 && hb < a.H) st16p<NT>(q + (int64_t)hb * a.q_head_stride + q_off1, hi);
                } else {
                    // k_pe second halves come from lanes 4..7 (all lanes take part)
                    const uint4 pe = buf[u][1];
                    uint4 pe_hi;
                    pe_hi.x = __shfl(pe.x, lane + 4, 64);
                    pe_hi.y = __shfl(pe.y, lane + 4, 64);
                    pe_hi.z = __shfl(pe.z, lane + 4, 64);
                    pe_hi.w = __shfl(pe.w, lane + 4, 64);
                    const int64_t row = s_row[ti];
                    if (pos >= 0 && row >= 0) {
                        kv_t* dst = cache + row;
                        if constexpr (KVFP8) {
                            float x[8];
                            unpack8(buf[u][0], x);
                            st8p<NT>(dst + 8 * lane, pack8_fp8(x, inv_scale));
                        } else {
                            st16p<NT>(dst + 8 * lane, buf[u][0]);
                        }
                        // latent ranks past the first 512 (kv_lora_rank = 1024, ...)
                        for (int e = 512 + 8 * lane; e < K; e += 512) {
                            const uint4 v = ld16(a.kv_c + (int64_t)t * a.kv_c_stride + e);
                            if constexpr (KVFP8) {
                                float x[8];
                                unpack8(v, x);
                                st8p<NT>(dst + e, pack8_fp8(x, inv_scale));
                            } else {
                                st16p<NT>(dst + e, v);
                            }
                        }
                        if (lane < kLanesPerHead) {
                            float c[8], s[8], x[16];
                            lane_cos_sin(s_cs + ti * kRope, gl, a.rope, c, s);
                            unpack8(pe, x);
                            unpack8(pe_hi, x + 8);
                            rope16(x, c, s, a.rope);
                            if constexpr (KVFP8) {
                                store_fp8_row<NT>(reinterpret_cast<uint8_t*>(dst + K), gl, kHalf, pack8_fp8(x, inv_scale),
                                              pack8_fp8(x + 8, inv_scale));
                            } else {
                                st16p<NT>(dst + K + 8 * gl, pack8_bf16(x));
                                st16p<NT>(dst + K + kHalf + 8 * gl, pack8_bf16(x + 8));
                            }
                        }
                    }
                }
                pr.advance(CPT);
            }
        }
    };

    for (bool first = true; sub_lo < bhi; first = false) {
        if (!first) __syncthreads();   // every wave is done with the previous tile's LDS
        start_tile();
        stage_tile();
        __syncthreads();
        inv_scale = KVFP8 ? 1.0f / kv_scale_v : 1.0f;
        while (pr.left > 0) {
            load_batch(bufB);
            run_batch(bufA);
            if (pr.left <= 0) break;
            load_batch(bufA);
            run_batch(bufB);
        }
        sub_lo = sub_hi;
    }
}

void set_divisors(MlaDevArgs& la) {
    la.grid_div = make_fastdiv31((uint32_t)la.grid);
    la.cpt_div = make_fastdiv31((uint32_t)(la.chunks_per_token > 0 ? la.chunks_per_token : 1));
    la.bs_div = make_fastdiv31((uint32_t)la.block_size);
    la.items_q = (int)(la.total_items / la.grid);
    la.items_r = (int)(la.total_items % la.grid);
}

template <bool KVFP8, bool NT>
hipError_t launch_t(const MlaDevArgs& a, hipStream_t stream) {
    MlaDevArgs la = a;
    // 8 (token, chunk) items per workgroup and no cap at the resident grid:
    // the dispatcher then hands the next workgroup to whichever CU finishes
    // first (4096 tokens x 128 heads: 4608 workgroups, 35.1 -> 33.5 us
    // against one range per resident workgroup; 4 items per workgroup
    // 36.5 us, 12 items 33.9 us)
    // (at most 32768 workgroups: the range split computes items_r * b with
    // items_r, b < grid in 31 bits)
    int64_t want = (a.total_items + 7) / 8;
    if (want < 1) want = 1;
    if (want > 32768) want = 32768;
    la.grid = (int)want;
    set_divisors(la);
    (void)hipGetLastError();   // the status below then covers this launch only
    hipLaunchKernelGGL((mla_kernel<KVFP8, NT>), dim3(la.grid), dim3(kBlockThreads), 0, stream, la);
    return hipGetLastError();
}

// ---------------------------------------------------------------------------
// FP8 Q modes: [q_nope | RoPE(q_rope)] -> E4M3 q_out (q read only) with a
// static per-tensor scale, or with one dynamic scale per token over all of
// its heads (vLLM issue: static per-tensor / dynamic per-token quantisation
// of the MLA query next to the FlashInfer MLA RoPE + quantize kernel).
//
// A workgroup takes whole tokens (t = blockIdx.x, + grid, ...), so the
// token's amax is one workgroup reduction (one barrier).  Four lanes own a
// head: lane l loads the NV = nope_dim / 32 nope vectors l, l + 4, ... (8
// elements each) and the rope vectors [8l, 8l+8), [32 + 8l, 32 + 8l + 8), so
// every load instruction covers 64 contiguous bytes of a head; a wave covers 16
// heads, a workgroup 64 per round, and two rounds (128 heads) are held in
// registers.  The token's cos/sin values are read straight into registers
// (every head uses the same 16 per lane).  One wave also writes the
// token's latent cache row.
// ---------------------------------------------------------------------------
constexpr int kQ8Rounds = 2;

template <int QMODE, bool KVFP8, bool NT>
__global__ __launch_bounds__(kBlockThreads) void mla_q8_kernel(const MlaDevArgs a) {
    typedef typename std::conditional<KVFP8, uint8_t, uint16_t>::type kv_t;
    __shared__ float s_amax[2][4];

    preload_kernargs(a);
    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);   // wave-uniform
    const int grp = lane / kLanesPerHead;
    const int gl = lane % kLanesPerHead;
    const int N = a.nope_dim;
    const int NV = N >> 5;
    const int K = a.kv_lora_rank;
    const int row_len = K + kRope;
    const int rounds = (a.H + 63) >> 6;
    const float q_static = (QMODE == 2) ? *a.q_scale_inv : 1.0f;
    const float inv_um = (QMODE == 1) ? 1.0f / a.upper_max : 1.0f;
    const float kv_scale_v = KVFP8 ? *a.kv_scale : 1.0f;   // reciprocal taken where first used
    kv_t* cache = reinterpret_cast<kv_t*>(a.kv_cache);
    int par = 0;   // s_amax slot: consecutive reductions alternate, so one barrier each suffices

    for (int64_t t = blockIdx.x; t < a.T; t += a.grid) {
        const int64_t pos = a.positions[t];
        if (pos < 0 || pos >= a.cs_rows) continue;     // suppressed token (same for the whole workgroup)
        const int64_t slot = a.slot_mapping[t];
        const uint16_t* qt = a.q + t * a.q_token_stride;
        uint8_t* ot = a.q_out + t * a.q_out_token_stride;
        const bool latent = wave == (int)(t & 3);
        uint4 kvv = make_uint4(0, 0, 0, 0), pe = make_uint4(0, 0, 0, 0);
        if (latent) {
            kvv = ld16(a.kv_c + t * a.kv_c_stride + 8 * lane);
            pe = ld16(a.k_pe + t * a.k_pe_stride + 8 * (lane & 7));
        }
        float c[8], s[8];
        lane_cos_sin(a.cos_sin + pos * kRope, gl, a.rope, c, s);

        for (int r0 = 0; r0 < rounds; r0 += kQ8Rounds) {
            uint4 vn[kQ8Rounds][4], vr[kQ8Rounds][2];
            int hh[kQ8Rounds];
#pragma unroll
            for (int k = 0; k < kQ8Rounds; ++k) {
                const int h = (r0 + k) * 64 + wave * kHeadsPerWave + grp;
                hh[k] = h;
                const uint16_t* qh = qt + (int64_t)(h < a.H ? h : 0) * a.q_head_stride;
                // nope vector j of lane gl: elements [8 (gl + 4 j), +8), so that
                // each load instruction reads 64 contiguous bytes of a head
                // (loading head pairs one whole line per instruction, as the
                // in-place kernel does, measured no faster here)
#pragma unroll
                for (int j = 0; j < 4; ++j) vn[k][j] = j < NV ? ld16(qh + 8 * (gl + 4 * j)) : make_uint4(0, 0, 0, 0);
                vr[k][0] = ld16(qh + N + 8 * gl);
                vr[k][1] = ld16(qh + N + kHalf + 8 * gl);
            }
            float xr[kQ8Rounds][16];
            float amax = 0.0f;
#pragma unroll
            for (int k = 0; k < kQ8Rounds; ++k) {
                unpack8(vr[k][0], xr[k]);
                unpack8(vr[k][1], xr[k] + 8);
                rope16(xr[k], c, s, a.rope);
                if (QMODE == 1 && hh[k] < a.H) {
#pragma unroll
                    for (int i = 0; i < 16; ++i) amax = __builtin_fmaxf(amax, __builtin_fabsf(xr[k][i]));
#pragma unroll
                    for (int j = 0; j < 4; ++j) {
                        float x[8];
                        unpack8(vn[k][j], x);   // zero vectors past NV
#pragma unroll
                        for (int i = 0; i < 8; ++i) amax = __builtin_fmaxf(amax, __builtin_fabsf(x[i]));
                    }
                }
            }
            float mul = q_static;
            if constexpr (QMODE == 1) {
                amax = group_max<16>(amax);
                amax = __builtin_fmaxf(amax, __shfl_xor(amax, 16, 64));
                amax = __builtin_fmaxf(amax, __shfl_xor(amax, 32, 64));
                if (lane == 0) s_amax[par][wave] = amax;
                __syncthreads();
                const float m = __builtin_fmaxf(__builtin_fmaxf(s_amax[par][0], s_amax[par][1]),
                                                __builtin_fmaxf(s_amax[par][2], s_amax[par][3]));
                par ^= 1;
                // s = max(amax, 1e-6) / upper_max; payload = v * (1 / s)
                const float sc = __builtin_fmaxf(m, 1e-6f) * inv_um;
                mul = __builtin_amdgcn_rcpf(sc);
                if (tid == 0) a.q_scale[t] = sc;
            }
#pragma unroll
            // (q_out rows take ordinary stores under either policy: each
            // instruction writes 64-byte pieces of the head rows, which L2
            // merges into whole lines; streamed, every piece went to memory
            // on its own: 27 % more bytes written and 65.0 against 62.2 us
            // on the 4096-token, 128-head workload with rotating buffers)
            for (int k = 0; k < kQ8Rounds; ++k) {
                if (hh[k] >= a.H) continue;   // whole 4-lane group skips together
                uint8_t* oh = ot + (int64_t)hh[k] * a.q_out_head_stride;
                if ((NV & 1) == 0) {
                    // codes of vectors j and j + 1 lie 32 bytes apart: neighbouring
                    // lanes trade one 8-byte piece and each stores 16 bytes
#pragma unroll
                    for (int j = 0; j < 4; j += 2) {
                        if (j < NV) {
                            float x[16];
                            unpack8(vn[k][j], x);
                            unpack8(vn[k][j + 1], x + 8);
                            store_fp8_row<false>(oh + 32 * j, gl, 32, pack8_fp8(x, mul), pack8_fp8(x + 8, mul));
                        }
                    }
                } else {
#pragma unroll
                    for (int j = 0; j < 4; ++j) {
                        if (j < NV) {
                            float x[8];
                            unpack8(vn[k][j], x);
                            st8(oh + 8 * (gl + 4 * j), pack8_fp8(x, mul));
                        }
                    }
                }
                store_fp8_row<false>(oh + N, gl, kHalf, pack8_fp8(xr[k], mul), pack8_fp8(xr[k] + 8, mul));
            }
        }

        if (latent) {
            // k_pe second halves come from lanes 4..7 (all lanes of the wave take part)
            uint4 pe_hi;
            pe_hi.x = __shfl(pe.x, lane + 4, 64);
            pe_hi.y = __shfl(pe.y, lane + 4, 64);
            pe_hi.z = __shfl(pe.z, lane + 4, 64);
            pe_hi.w = __shfl(pe.w, lane + 4, 64);
            if (slot >= 0 && slot < a.capacity) {
                kv_t* dst = cache + cache_row(a, slot, row_len);
                if constexpr (KVFP8) {
                    float x[8];
                    unpack8(kvv, x);
                    st8p<NT>(dst + 8 * lane, pack8_fp8(x, 1.0f / kv_scale_v));
                } else {
                    st16p<NT>(dst + 8 * lane, kvv);
                }
                for (int e = 512 + 8 * lane; e < K; e += 512) {
                    const uint4 v = ld16(a.kv_c + t * a.kv_c_stride + e);
                    if constexpr (KVFP8) {
                        float x[8];
                        unpack8(v, x);
                        st8p<NT>(dst + e, pack8_fp8(x, 1.0f / kv_scale_v));
                    } else {
                        st16p<NT>(dst + e, v);
                    }
                }
                if (lane < kLanesPerHead) {
                    float x[16];
                    unpack8(pe, x);
                    unpack8(pe_hi, x + 8);
                    rope16(x, c, s, a.rope);
                    if constexpr (KVFP8) {
                        store_fp8_row<NT>(reinterpret_cast<uint8_t*>(dst + K), gl, kHalf,
                                      pack8_fp8(x, 1.0f / kv_scale_v), pack8_fp8(x + 8, 1.0f / kv_scale_v));
                    } else {
                        st16p<NT>(dst + K + 8 * gl, pack8_bf16(x));
                        st16p<NT>(dst + K + kHalf + 8 * gl, pack8_bf16(x + 8));
                    }
                }
            }
        }
    }
}

template <int QMODE, bool KVFP8, bool NT>
hipError_t launch_q8_t(const MlaDevArgs& a, hipStream_t stream) {
    MlaDevArgs la = a;
    int64_t cap = resident_grid(reinterpret_cast<const void*>(&mla_q8_kernel<QMODE, KVFP8, NT>), 0);
    if (cap < 1) cap = 256;
    // twice the resident grid: a workgroup that finishes its tokens early is
    // replaced by one that has not started (4096 tokens x 128 heads: static
    // scale 61.9 -> 60.4 us, dynamic 61.9 -> 61.5 us; 8x the resident grid
    // was slower for the dynamic scale)
    cap *= 2;
    la.grid = (int)(a.T < cap ? a.T : cap);
    set_divisors(la);
    (void)hipGetLastError();   // the status below then covers this launch only
    hipLaunchKernelGGL((mla_q8_kernel<QMODE, KVFP8, NT>), dim3(la.grid), dim3(kBlockThreads), 0, stream, la);
    return hipGetLastError();
}

}  // namespace

hipError_t launch_mla_concat_rope(const MlaDevArgs& a, int kv_fp8, hipStream_t stream) {
    if (a.nt_store) return kv_fp8 ? launch_t<true, true>(a, stream) : launch_t<false, true>(a, stream);
    return kv_fp8 ? launch_t<true, false>(a, stream) : launch_t<false, false>(a, stream);
}

hipError_t launch_mla_q8(const MlaDevArgs& a, int kv_fp8, hipStream_t stream) {
    const bool nt = a.nt_store != 0;
    if (a.q_mode == 1) {
        if (nt) return kv_fp8 ? launch_q8_t<1, true, true>(a, stream) : launch_q8_t<1, false, true>(a, stream);
        return kv_fp8 ? launch_q8_t<1, true, false>(a, stream) : launch_q8_t<1, false, false>(a, stream);
    }
    if (nt) return kv_fp8 ? launch_q8_t<2, true, true>(a, stream) : launch_q8_t<2, false, true>(a, stream);
    return kv_fp8 ? launch_q8_t<2, true, false>(a, stream) : launch_q8_t<2, false, false>(a, stream);
}

}  // namespace qkprep
