/*
 * qkprep.h -- C ABI of libqkprep, the fused pre-attention "prepare" pass for
 * MI355X (gfx950).
 *
 * One call makes a single pass over a packed (or strided) bf16 QKV
 * activation and, per token: normalises each Q and K head (RMSNorm or the
 * Gemma (1 + w) variant), rotates it with RoPE from an fp32 cos/sin table
 * indexed by the token's int64 position, encodes Q (bf16, or FP8 E4M3 with
 * a dynamic per-token-per-head or a static scale), and appends K and V to a
 * paged NHD cache through a page table or a slot mapping, clearing the tail
 * of each request's last page.  A second entry point does the MLA variant:
 * RoPE on the rope slice of q in place and the [latent | rope(k_pe)] concat
 * into a latent cache.
 *
 * Where the operations are defined (the pages):
 *  - FlashInfer PR "fused QK RMSNorm + NeoX RoPE + FP8 E4M3 quantize + NHD
 *    paged-KV append", sections "What changes" and "Contract": argument set,
 *    packed qkv [T, (Hq + 2 Hkv) * D], NHD caches, q_scale layouts, K/V as
 *    x / scale, RN-satfinite FP8, upper_max in (0, 448], seq_lens after the
 *    append, tail clear, all-or-nothing validation on the device without a
 *    host sync, one launch per call; its review threads (empty batch returns
 *    without a launch, page_size <= 0 rejected, seq_len < q_len and page
 *    overflow as invalid metadata).
 *  - TensorRT-LLM PR "Fuse Qwen3.5 gated QKV preprocessing", Phase 1/2:
 *    strided QKV rows, Gemma Q/K RMSNorm folded into the KV-append pass.
 *  - SGLang PR "fused Q/K RMSNorm + RoPE with cos_sin_cache": fp32
 *    cos_sin_cache, 1-D int64 positions, strided views into packed QKV.
 *  - vLLM issue "ROPE + KV-Cache-Write + pre-attn prepare-ops fusion":
 *    reshape_and_cache slot scatter and concat_and_cache_mla.
 *
 * Conventions for every entry point:
 *  - All array pointers are DEVICE pointers owned by the caller; the params
 *    struct itself is a host pointer read during the call only.  The library
 *    allocates nothing, keeps no state between calls, never synchronises the
 *    stream and never reads device memory on the host, so a call is safe to
 *    capture in a HIP graph.  Work is enqueued on `stream` (0 = the null
 *    stream) and the status only covers the host-side checks and the launch.
 *  - Strides and offsets are in ELEMENTS of the array they index.
 *  - Every base address and row stride that the kernels load or store in
 *    16-byte vectors must be 16-byte aligned (see each field); otherwise the
 *    call returns QKPREP_E_ALIGN before launching.
 *  - Invalid arguments detectable on the host return a non-zero status and
 *    enqueue nothing.  Invalid request metadata is detected on the device:
 *    every flags[b][h] becomes -1 and no other byte is written.
 */
#ifndef QKPREP_H
#define QKPREP_H

#include <stdint.h>
#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

#define QKPREP_ABI_VERSION 2

typedef enum {
    QKPREP_OK = 0,
    QKPREP_E_NULL = 1,         /* a required pointer is NULL */
    QKPREP_E_SHAPE = 2,        /* inconsistent sizes or strides */
    QKPREP_E_UNSUPPORTED = 3,  /* a valid configuration the library does not implement */
    QKPREP_E_ALIGN = 4,        /* a vector-accessed base or stride is not 16-byte aligned */
    QKPREP_E_RANGE = 5,        /* a scalar outside its documented range */
    QKPREP_E_LAUNCH = 6,       /* the HIP launch itself failed */
    QKPREP_E_VERSION = 7       /* struct_size does not match this library */
} qkprep_status;

typedef enum { QKPREP_BF16 = 0, QKPREP_FP8_E4M3 = 1 } qkprep_dtype;
typedef enum { QKPREP_NORM_NONE = 0, QKPREP_NORM_RMS = 1, QKPREP_NORM_GEMMA = 2 } qkprep_norm;
typedef enum { QKPREP_ROPE_NEOX = 0, QKPREP_ROPE_INTERLEAVED = 1 } qkprep_rope;
typedef enum {
    QKPREP_Q_BF16 = 0,         /* Q stored as bf16 (RNE) */
    QKPREP_Q_FP8_DYNAMIC = 1,  /* per-(token, head) scale s = max(amax, 1e-6) / upper_max */
    QKPREP_Q_FP8_STATIC = 2    /* payload = q * q_scale_inv */
} qkprep_qmode;
typedef enum {
    QKPREP_QSCALE_TOKEN_HEAD = 0,     /* q_scale[t][h]                                       */
    QKPREP_QSCALE_REQ_HEAD_PADDED = 1 /* q_scale[b][h][j], j = token index inside request b,  */
                                      /* row length P = round_up(max_seqlen, 128)             */
} qkprep_qscale_layout;
typedef enum { QKPREP_ADDR_PAGED = 0, QKPREP_ADDR_SLOT = 1 } qkprep_addressing;
/* Cache policy for the rows a call writes (token rows of Q, K and V, the MLA
 * latent rows and the E4M3 MLA query).  Not on the pages, which leave the
 * store path open; a choice of this library, measured on MI355X. */
typedef enum {
    QKPREP_STORE_STREAM = 0,   /* default: non-temporal stores for the long contiguous rows (Q
                                  rows, the MLA latent rows and rope slices), so that they drain
                                  to HBM as they are produced instead of occupying L2 and the
                                  Infinity Cache; K/V cache rows of the norm-rope-append call
                                  and rows written back into qkv (in-place Q / K) keep ordinary
                                  stores (measured faster for those) */
    QKPREP_STORE_KEEP = 1      /* ordinary stores everywhere: the rows stay in L2 / the
                                  Infinity Cache for a kernel that reads them right after */
} qkprep_store_policy;
typedef enum {
    QKPREP_KV_SCALE_STATIC = 0,    /* device scalars k_scale / v_scale */
    QKPREP_KV_SCALE_TOKEN = 1,     /* dynamic, one per (token, kv head) */
    QKPREP_KV_SCALE_GROUP = 2      /* dynamic, one per kv_group_size consecutive dims */
} qkprep_kv_scale_mode;

/*
 * qkprep_norm_rope_append -- Q/K RMSNorm + RoPE + (FP8) quantisation + paged
 * KV append.  FlashInfer PR "fused QK RMSNorm + NeoX RoPE + FP8 E4M3 quantize
 * + NHD paged-KV append", "Contract"; TensorRT-LLM PR "Fuse Qwen3.5 gated QKV
 * preprocessing", Phase 2; SGLang PR "fused Q/K RMSNorm + RoPE with
 * cos_sin_cache", "Modifications".
 *
 * For each token t of request b (tokens q_indptr[b] .. q_indptr[b+1]-1,
 * j = t - q_indptr[b], q_len = q_indptr[b+1] - q_indptr[b]):
 *   x     = head row of qkv (bf16 -> fp32)
 *   y     = x * rsqrt(mean(x^2) + eps) * w      (norm RMS; w -> 1 + w for GEMMA)
 *   o     = RoPE(y) on the first R = rotary_dim dims, with
 *           c_i = cos_sin[pos][i], s_i = cos_sin[pos][R/2 + i];
 *           NEOX pairs (i, i + R/2), INTERLEAVED pairs (2i, 2i + 1), i < R/2:
 *           (a, b) -> (a c - b s, b c + a s); dims [R, D) pass through
 *           (partial rotary, vLLM issue's model table: RoPE on part of the
 *           head, NoPE on the rest; R = 0 is a NoPE layer)
 *   Q     -> q_out[t][h] : bf16(o), or E4M3(o / s) with s stored in q_scale,
 *            or E4M3(o * q_scale_inv)
 *   K     -> cache row  : bf16(o) or E4M3(o / k_scale); optionally bf16(o) to k_out
 *   V     -> cache row  : raw bf16 bits or E4M3(x / v_scale)
 * Paged addressing: L = seq_lens[b] - q_len + j, page = page_table[b][L / ps],
 * row = L % ps.  Slot addressing: page = slot / ps, row = slot % ps.
 * E4M3 is OCP E4M3FN, round to nearest even, finite overflow saturates to
 * +-448.  Positions outside [0, cos_sin_rows) suppress the whole token (no
 * byte written for it); with rotary_dim 0 positions and the table are not
 * read and nothing is suppressed.
 *
 * Device validation (paged addressing only), all-or-nothing: the call is
 * invalid if q_indptr[0] != 0, q_indptr[B] != T, q_indptr decreases,
 * seq_lens[b] < q_len, seq_lens[b] > max_pages_per_request * page_size, a
 * page this call writes has an id outside [0, num_pages), or (padded
 * q_scale layout) q_len > max_seqlen.  An invalid call writes flags[b][h] =
 * -1 for every (b, h) and nothing else; a valid call writes flags = 0.
 * Tail clear (zero_tail != 0, paged only): rows [last + 1, page_size) of the
 * page holding logical row seq_lens[b] - 1 are set to zero bytes in both
 * caches for every request with seq_lens[b] > 0 (empty requests included).
 */
typedef struct qkprep_norm_rope_append_params {
    uint32_t struct_size;          /* = sizeof(qkprep_norm_rope_append_params) */

    int32_t num_tokens;            /* T >= 0; T * ceil((Hq + 2 Hkv) / (64 / (D / 16))) < 2^31 */
    int32_t num_q_heads;           /* Hq >= 1 */
    int32_t num_kv_heads;          /* Hkv >= 1, Hq % Hkv == 0 */
    int32_t head_dim;              /* D: 64, 128 or 256 */
    int32_t rotary_dim;            /* R: rotated dims, 0 <= R <= D, multiple of 16 (R = D: whole head) */

    const void* qkv;               /* bf16 [T][qkv_row_stride]; heads Q(Hq) | K(Hkv) | V(Hkv), 16-B aligned */
    int64_t qkv_row_stride;        /* >= (Hq + 2 Hkv) * D, multiple of 8 */

    int32_t norm;                  /* qkprep_norm */
    float eps;                     /* > 0 when norm != NONE (1e-6 in the pages) */
    const float* q_norm_weight;    /* fp32 [D], 16-B aligned; required when norm != NONE */
    const float* k_norm_weight;    /* fp32 [D], 16-B aligned; required when norm != NONE */

    int32_t rope;                  /* qkprep_rope */
    const float* cos_sin_cache;    /* fp32 [cos_sin_rows][rotary_dim]: cos half | sin half, 16-B aligned;
                                      not read (may be NULL) when rotary_dim == 0 */
    int64_t cos_sin_rows;          /* >= 1 when rotary_dim > 0 */
    const int64_t* positions;      /* int64 [T]; not read (may be NULL) when rotary_dim == 0 */

    int32_t addressing;            /* qkprep_addressing */
    int32_t num_requests;          /* B; paged: 0 <= B <= 4096 (and B >= 1 when T > 0); slot: ignored */
    const int32_t* q_indptr;       /* int32 [B + 1] (paged) */
    const int32_t* seq_lens;       /* int32 [B], length after the append (paged) */
    const int32_t* page_table;     /* int32 [B][max_pages_per_request] (paged) */
    int32_t max_pages_per_request; /* >= 1 (paged) */
    const int64_t* slot_mapping;   /* int64 [T] (slot); slot < 0 or >= num_pages * page_size skips K/V */

    void* k_cache;                 /* [num_pages][page_size][Hkv][D] of kv_dtype, 16-B aligned */
    void* v_cache;                 /* same shape, may have its own page stride */
    int32_t kv_dtype;              /* qkprep_dtype */
    int32_t num_pages;             /* >= 1 */
    int32_t page_size;             /* >= 1 */
    int64_t k_page_stride;         /* elements between pages, >= page_size * Hkv * D, 16-B multiple */
    int64_t v_page_stride;
    const float* k_scale;          /* device fp32 scalar (FP8 cache, static scales only) */
    const float* v_scale;          /* device fp32 scalar (FP8 cache, static scales only) */
    int32_t zero_tail;             /* paged only; 1 in the pages' contract */

    void* q_out;                   /* [T][q_out_row_stride]: bf16 (Q_BF16) or E4M3 codes; may be
                                      exactly qkv (same base and stride) for Q in place (bf16 only) */
    int64_t q_out_row_stride;      /* >= Hq * D; bf16: multiple of 8, FP8: multiple of 16 */
    int32_t q_mode;                /* qkprep_qmode */
    float* q_scale;                /* FP8_DYNAMIC: fp32, layout per q_scale_layout */
    int32_t q_scale_layout;        /* qkprep_qscale_layout (FP8_DYNAMIC) */
    int32_t max_seqlen;            /* >= 1 for the padded layout */
    const float* q_scale_inv;      /* FP8_STATIC: device fp32 scalar */
    float upper_max;               /* FP8_DYNAMIC: finite, in (0, 448] */

    void* k_out;                   /* optional bf16 [T][k_out_row_stride] roped K; may be exactly the K
                                      columns of qkv (qkv + Hq*D elements, same stride) */
    int64_t k_out_row_stride;      /* >= Hkv * D, multiple of 8 */

    int32_t* flags;                /* int32 [B][Hkv] (paged); may be NULL when B == 0 */

    /* K/V redirect (FlashInfer PR "Contract": caller-owned out_k / out_v; its
     * review: no tail clear when K/V are redirected).  With out_k and out_v
     * set, the K and V rows of token t go to out_k[t][h][:] / out_v[t][h][:]
     * (kv_dtype, same encoding as a cache row) instead of the caches; the
     * caches are neither read nor written (they and the slot mapping may be
     * NULL), zero_tail is ignored, and the paged metadata is validated as
     * usual (flags). */
    void* out_k;                   /* [T][out_kv_row_stride] of kv_dtype, 16-B aligned; NULL = no redirect */
    void* out_v;                   /* set together with out_k */
    int64_t out_kv_row_stride;     /* >= Hkv * D elements, 16-B multiple */

    /* FP8 K/V scales (vLLM issue: static per-tensor, dynamic per-token and
     * dynamic per-group quantisation).  Dynamic modes encode each group of g
     * dims (g = D per token, else kv_group_size) as E4M3(x / s) with
     * s = max(max |x| over the group, 1e-6) / 448 (x: K after norm + RoPE, V
     * raw) and store s at k_scale_out / v_scale_out, fp32
     * [num_pages * page_size][Hkv][D / g] indexed by the cache row
     * page * page_size + row (or [T][Hkv][D / g] by token with out_k / out_v).
     * A cleared tail row gets zero scales.  Needs the FP8 cache; GROUP needs
     * kv_group_size a power of two in [8, D/2] (or D), and a group smaller
     * than the head needs rotary_dim == D or 0. */
    int32_t kv_scale_mode;         /* qkprep_kv_scale_mode */
    int32_t kv_group_size;
    float* k_scale_out;
    float* v_scale_out;

    int32_t store_policy;          /* qkprep_store_policy (0 = QKPREP_STORE_STREAM) */
} qkprep_norm_rope_append_params;

/*
 * qkprep_mla_concat_rope_append -- MLA latent cache append.  vLLM issue
 * "ROPE + KV-Cache-Write + pre-attn prepare-ops fusion" (concat_and_cache_mla,
 * concat_cache_mla_rope; DeepSeek-R1 row of the model table: 128 heads,
 * 64 rope + 128 nope dims, latent 512).
 *
 * For each token t with position pos in [0, cos_sin_rows) (others write
 * nothing):
 *   q[t][h][nope_dim : nope_dim + rope_dim] <- bf16(RoPE(that slice)), in place
 *   if 0 <= slot_mapping[t] < num_blocks * block_size, the cache row
 *   cache[slot / block_size][slot % block_size][0 : kv_lora_rank + rope_dim]
 *   <- [kv_c[t] | RoPE(k_pe[t])] as E4M3(x / kv_scale) (FP8 cache) or as
 *      bf16 (kv_c bits copied, RoPE result rounded).
 * k_pe is read only.  RoPE pairs follow `rope` as above, angle i uses
 * cos_sin[pos][i] and cos_sin[pos][rope_dim/2 + i].
 */
typedef struct qkprep_mla_params {
    uint32_t struct_size;          /* = sizeof(qkprep_mla_params) */

    int32_t num_tokens;            /* T >= 0; T * (ceil(H / 16) + 1) < 2^31 */
    int32_t num_q_heads;           /* H >= 1 */
    int32_t nope_dim;              /* >= 0, multiple of 8 */
    int32_t rope_dim;              /* 64 */
    int32_t kv_lora_rank;          /* multiple of 512 */

    void* q;                       /* bf16, element (t, h, d) at t*q_token_stride + h*q_head_stride + d */
    int64_t q_token_stride;        /* multiples of 8; rope slice of each head 16-B aligned */
    int64_t q_head_stride;

    const void* kv_c;              /* bf16 [T][kv_c_stride] */
    int64_t kv_c_stride;           /* >= kv_lora_rank, multiple of 8 */
    const void* k_pe;              /* bf16 [T][k_pe_stride] */
    int64_t k_pe_stride;           /* >= rope_dim, multiple of 8 */

    int32_t rope;                  /* qkprep_rope (DeepSeek: INTERLEAVED) */
    const float* cos_sin_cache;    /* fp32 [cos_sin_rows][rope_dim] */
    int64_t cos_sin_rows;
    const int64_t* positions;      /* int64 [T] */
    const int64_t* slot_mapping;   /* int64 [T]; out-of-range slot skips the cache write */

    void* kv_cache;                /* [num_blocks][block_size][kv_lora_rank + rope_dim] of kv_dtype */
    int32_t kv_dtype;              /* qkprep_dtype */
    int64_t num_blocks;            /* >= 1 */
    int32_t block_size;            /* >= 1 */
    int64_t block_stride;          /* elements, >= block_size * (kv_lora_rank + rope_dim) */
    const float* kv_scale;         /* device fp32 scalar (FP8 cache only) */

    /* Q output.  Q_BF16: RoPE in place in q as above (the fields below are
     * unused).  FP8_STATIC / FP8_DYNAMIC: q is read only and
     *   q_out[t][h][0 : nope_dim + rope_dim] <- E4M3(v * q_scale_inv)      (static)
     *                                        or E4M3(v / s_t)             (dynamic)
     * with v = [q_nope | RoPE(q_rope)] in fp32 and, per token, one scale
     * s_t = max(max |v| over all heads and dims, 1e-6) / upper_max stored at
     * q_scale[t].  Needs nope_dim a multiple of 32 and at most 128; the
     * dynamic mode needs num_q_heads <= 128.  A suppressed token writes
     * neither q_out nor q_scale. */
    int32_t q_mode;                /* qkprep_qmode */
    void* q_out;                   /* E4M3 codes, (t, h, d) at t*q_out_token_stride + h*q_out_head_stride + d;
                                      16-B aligned, must not overlap q */
    int64_t q_out_token_stride;    /* multiple of 16 */
    int64_t q_out_head_stride;     /* >= nope_dim + rope_dim, multiple of 16 */
    float* q_scale;                /* FP8_DYNAMIC: fp32 [T] */
    const float* q_scale_inv;      /* FP8_STATIC: device fp32 scalar */
    float upper_max;               /* FP8_DYNAMIC: finite, in (0, 448] */

    int32_t store_policy;          /* qkprep_store_policy (0 = QKPREP_STORE_STREAM); the latent rows
                                      and the in-place q rope slices follow it; the E4M3 q_out rows
                                      always take ordinary stores (written in 64-byte pieces that L2
                                      merges into whole lines) */
} qkprep_mla_params;

/* Host checks, then one kernel launch on `stream` (none when there is no
 * work).  Returns QKPREP_OK or the first failing check. */
qkprep_status qkprep_norm_rope_append(const qkprep_norm_rope_append_params* params, hipStream_t stream);

/* Host checks, then one kernel launch on `stream` (none when T == 0). */
qkprep_status qkprep_mla_concat_rope_append(const qkprep_mla_params* params, hipStream_t stream);

/* Static English text for a status code; never NULL. */
const char* qkprep_status_string(qkprep_status status);

/* QKPREP_ABI_VERSION of the built library. */
int qkprep_abi_version(void);

#ifdef __cplusplus
}
#endif

#endif /* QKPREP_H */
