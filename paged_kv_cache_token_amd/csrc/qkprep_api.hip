// C-ABI entry points of libqkprep: host-side argument checks, the empty-call
// early return, launch-geometry choice and the single kernel launch.
//
// Host guards follow the review threads of the FlashInfer PR "fused QK
// RMSNorm + NeoX RoPE + FP8 E4M3 quantize + NHD paged-KV append": an empty
// batch returns without a launch, page_size <= 0 is rejected, invalid
// upper_max / quant policy is rejected.  Nothing here reads device memory.
#include <math.h>
#include <stdint.h>

#include <mutex>
#include <vector>

#include "qkprep.h"
#include "qkprep_internal.h"

using namespace qkprep;

namespace {

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

struct ResidentEntry {
    const void* kernel;
    int device;
    size_t lds;
    int grid;
};

}  // namespace

namespace qkprep {

int resident_grid(const void* kernel, size_t dyn_lds) {
    static std::mutex mu;
    static std::vector<ResidentEntry> cache;
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess) {
        (void)hipGetLastError();
        return 0;
    }
    {
        std::lock_guard<std::mutex> lock(mu);
        for (const ResidentEntry& e : cache)
            if (e.kernel == kernel && e.device == dev && e.lds == dyn_lds) return e.grid;
    }
    int per_cu = 0, cus = 0;
    if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&per_cu, kernel, kBlockThreads, dyn_lds) != hipSuccess ||
        hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess) {
        (void)hipGetLastError();
        return 0;
    }
    const int grid = (per_cu < 1 ? 1 : per_cu) * (cus < 1 ? 1 : cus);
    std::lock_guard<std::mutex> lock(mu);
    cache.push_back(ResidentEntry{kernel, dev, dyn_lds, grid});
    return grid;
}

}  // namespace qkprep

extern "C" {

const char* qkprep_status_string(qkprep_status status) {
    switch (status) {
        case QKPREP_OK: return "ok";
        case QKPREP_E_NULL: return "a required pointer is NULL";
        case QKPREP_E_SHAPE: return "inconsistent sizes or strides";
        case QKPREP_E_UNSUPPORTED: return "configuration not supported by this library";
        case QKPREP_E_ALIGN: return "a vector-accessed base address or stride is not 16-byte aligned";
        case QKPREP_E_RANGE: return "a scalar argument is outside its documented range";
        case QKPREP_E_LAUNCH: return "the HIP kernel launch failed";
        case QKPREP_E_VERSION: return "params.struct_size does not match this library";
    }
    return "unknown status";
}

int qkprep_abi_version(void) { return QKPREP_ABI_VERSION; }

qkprep_status qkprep_norm_rope_append(const qkprep_norm_rope_append_params* p, hipStream_t stream) {
    if (!p) return QKPREP_E_NULL;
    if (p->struct_size != sizeof(qkprep_norm_rope_append_params)) return QKPREP_E_VERSION;
    const int T = p->num_tokens, Hq = p->num_q_heads, Hkv = p->num_kv_heads, D = p->head_dim;
    if (T < 0 || Hq < 1 || Hkv < 1 || Hq % Hkv != 0) return QKPREP_E_SHAPE;
    if (D != 64 && D != 128 && D != 256) return QKPREP_E_UNSUPPORTED;
    const int rot = p->rotary_dim;
    if (rot < 0 || rot > D || rot % 16) return QKPREP_E_UNSUPPORTED;
    if (p->norm < 0 || p->norm > 2 || p->rope < 0 || p->rope > 1 || p->addressing < 0 ||
        p->addressing > 1 || p->kv_dtype < 0 || p->kv_dtype > 1 || p->q_mode < 0 || p->q_mode > 2 ||
        p->q_scale_layout < 0 || p->q_scale_layout > 1)
        return QKPREP_E_RANGE;
    if (p->page_size <= 0) return QKPREP_E_RANGE;
    if (p->store_policy < 0 || p->store_policy > 1) return QKPREP_E_RANGE;
    const bool redirect = p->out_k != nullptr || p->out_v != nullptr;
    if (redirect && (!p->out_k || !p->out_v)) return QKPREP_E_NULL;
    if (p->kv_scale_mode < 0 || p->kv_scale_mode > 2) return QKPREP_E_RANGE;
    const bool kv_dyn = p->kv_scale_mode != QKPREP_KV_SCALE_STATIC;
    int kv_group = 0;
    if (kv_dyn) {
        if (p->kv_dtype != QKPREP_FP8_E4M3) return QKPREP_E_UNSUPPORTED;
        kv_group = D;
        if (p->kv_scale_mode == QKPREP_KV_SCALE_GROUP) {
            const int g = p->kv_group_size;
            if (g < 8 || (g & (g - 1)) || (g > D / 2 && g != D)) return QKPREP_E_UNSUPPORTED;
            // groups inside a head need the whole-head lane layout, which
            // calls rotating all dims or none use
            if (g != D && rot != D && rot != 0) return QKPREP_E_UNSUPPORTED;
            kv_group = g;
        }
    }
    if (p->norm != 0 && !(p->eps > 0.0f && isfinite(p->eps))) return QKPREP_E_RANGE;
    if (p->q_mode == QKPREP_Q_FP8_DYNAMIC && !(p->upper_max > 0.0f && p->upper_max <= 448.0f))
        return QKPREP_E_RANGE;
    const bool paged = p->addressing == QKPREP_ADDR_PAGED;
    const int B = paged ? p->num_requests : 0;
    const bool padded = p->q_mode == QKPREP_Q_FP8_DYNAMIC && p->q_scale_layout == QKPREP_QSCALE_REQ_HEAD_PADDED;
    if (paged) {
        if (B < 0) return QKPREP_E_SHAPE;
        if (T > 0 && B == 0) return QKPREP_E_SHAPE;
        if (B > kMaxRequests) return QKPREP_E_UNSUPPORTED;
    } else if (padded) {
        return QKPREP_E_UNSUPPORTED;   // the padded layout is indexed by request
    }
    if (padded && p->max_seqlen < 1) return QKPREP_E_RANGE;
    // empty batch: nothing to write, no launch
    if (T == 0 && B == 0) return QKPREP_OK;

    const int R = Hq + 2 * Hkv;
    const int kv_elt = p->kv_dtype == QKPREP_FP8_E4M3 ? 1 : 2;
    const int q_elt = p->q_mode == QKPREP_Q_BF16 ? 2 : 1;
    // pointers
    if (!redirect && (!p->k_cache || !p->v_cache)) return QKPREP_E_NULL;
    if (p->kv_dtype == QKPREP_FP8_E4M3 && !kv_dyn && (!p->k_scale || !p->v_scale)) return QKPREP_E_NULL;
    if (kv_dyn && (!p->k_scale_out || !p->v_scale_out)) return QKPREP_E_NULL;
    if (paged && (!p->q_indptr || !p->seq_lens || !p->page_table || !p->flags)) return QKPREP_E_NULL;
    if (T > 0) {
        if (!p->qkv || !p->q_out) return QKPREP_E_NULL;
        if (rot > 0 && (!p->cos_sin_cache || !p->positions)) return QKPREP_E_NULL;
        if (p->norm != 0 && (!p->q_norm_weight || !p->k_norm_weight)) return QKPREP_E_NULL;
        if (!paged && !redirect && !p->slot_mapping) return QKPREP_E_NULL;
        if (p->q_mode == QKPREP_Q_FP8_DYNAMIC && !p->q_scale) return QKPREP_E_NULL;
        if (p->q_mode == QKPREP_Q_FP8_STATIC && !p->q_scale_inv) return QKPREP_E_NULL;
    }
    // sizes and strides
    if (p->num_pages < 1) return QKPREP_E_SHAPE;
    if (paged && p->max_pages_per_request < 1) return QKPREP_E_SHAPE;
    const int64_t row_elems = (int64_t)Hkv * D;
    if (redirect) {
        if (p->out_kv_row_stride < row_elems) return QKPREP_E_SHAPE;
        if ((p->out_kv_row_stride * kv_elt) % 16 || !aligned16(p->out_k) || !aligned16(p->out_v))
            return QKPREP_E_ALIGN;
    } else {
        if (p->k_page_stride < (int64_t)p->page_size * row_elems ||
            p->v_page_stride < (int64_t)p->page_size * row_elems)
            return QKPREP_E_SHAPE;
        if ((p->k_page_stride * kv_elt) % 16 || (p->v_page_stride * kv_elt) % 16) return QKPREP_E_ALIGN;
        if (!aligned16(p->k_cache) || !aligned16(p->v_cache)) return QKPREP_E_ALIGN;
    }
    if (T > 0) {
        if (p->qkv_row_stride < (int64_t)R * D) return QKPREP_E_SHAPE;
        if (p->qkv_row_stride % 8) return QKPREP_E_ALIGN;
        if (p->q_out_row_stride < (int64_t)Hq * D) return QKPREP_E_SHAPE;
        if ((p->q_out_row_stride * q_elt) % 16) return QKPREP_E_ALIGN;
        if (rot > 0 && p->cos_sin_rows < 1) return QKPREP_E_SHAPE;
        if (!aligned16(p->qkv) || !aligned16(p->q_out)) return QKPREP_E_ALIGN;
        if (rot > 0 && !aligned16(p->cos_sin_cache)) return QKPREP_E_ALIGN;
        if (p->norm != 0 && (!aligned16(p->q_norm_weight) || !aligned16(p->k_norm_weight)))
            return QKPREP_E_ALIGN;
        if (p->k_out) {
            if (p->k_out_row_stride < row_elems) return QKPREP_E_SHAPE;
            if (p->k_out_row_stride % 8 || !aligned16(p->k_out)) return QKPREP_E_ALIGN;
        }
    }

    NraDevArgs a{};
    a.T = T; a.Hq = Hq; a.Hkv = Hkv; a.R = R;
    a.qkv = static_cast<const uint16_t*>(p->qkv);
    a.qkv_stride = p->qkv_row_stride;
    a.norm = p->norm; a.eps = p->eps;
    a.q_w = p->q_norm_weight; a.k_w = p->k_norm_weight;
    a.rope = p->rope;
    a.rot = rot;
    a.cos_sin = rot > 0 ? p->cos_sin_cache : nullptr;
    a.cs_rows = rot > 0 ? p->cos_sin_rows : 0;
    a.positions = rot > 0 ? p->positions : nullptr;
    a.paged = paged ? 1 : 0;
    a.B = B;
    a.q_indptr = p->q_indptr; a.seq_lens = p->seq_lens; a.page_table = p->page_table;
    a.maxp = p->max_pages_per_request;
    a.pt_vec = paged && !redirect && B <= kSearchRequests && aligned16(p->page_table) &&
                       p->max_pages_per_request % 4 == 0
                   ? 1
                   : 0;
    a.slot_mapping = p->slot_mapping;
    a.k_cache = redirect ? p->out_k : p->k_cache;
    a.v_cache = redirect ? p->out_v : p->v_cache;
    a.redirect = redirect ? 1 : 0;
    a.kv_out_stride = redirect ? p->out_kv_row_stride : 0;
    a.kv_group = kv_group;
    a.k_scale_out = p->k_scale_out; a.v_scale_out = p->v_scale_out;
    a.num_pages = p->num_pages; a.page_size = p->page_size;
    a.ps_div = make_fastdiv31((uint32_t)p->page_size);
    a.k_page_stride = p->k_page_stride; a.v_page_stride = p->v_page_stride;
    a.k_scale = p->k_scale; a.v_scale = p->v_scale;
    a.zero_tail = paged && !redirect && p->zero_tail ? 1 : 0;
    a.q_out = p->q_out; a.q_out_stride = p->q_out_row_stride;
    a.q_scale = p->q_scale;
    a.q_scale_padded = padded ? 1 : 0;
    a.max_seqlen = p->max_seqlen;
    a.q_scale_P = padded ? ((int64_t)p->max_seqlen + 127) / 128 * 128 : 0;
    a.stage_q_scale = padded && Hq <= kMaxStagedQHeads ? 1 : 0;
    a.q_scale_inv = p->q_scale_inv;
    a.upper_max = p->upper_max;
    a.k_out = static_cast<uint16_t*>(p->k_out);
    // qkv rows are read once unless Q or K is written back into them; the
    // rows written back keep ordinary stores (measured faster there)
    const bool in_place = p->q_out == p->qkv || p->k_out != nullptr;
    a.mem = in_place ? kMemInPlace : (p->store_policy == QKPREP_STORE_KEEP ? kMemKeep : kMemStream);
    a.k_out_stride = p->k_out_row_stride;
    a.flags = p->flags;
    const int rows_per_wave = 64 / (D / 16);
    a.chunks_per_token = (R + rows_per_wave - 1) / rows_per_wave;
    a.tokens_per_tile = kMaxTokensPerTile;
    a.total_items = (int64_t)T * a.chunks_per_token;
    // the kernel indexes (token, chunk) items with 32-bit integers
    if (a.total_items > INT32_MAX) return QKPREP_E_SHAPE;

    hipError_t e = launch_norm_rope_append(a, D, p->q_mode, p->kv_dtype, stream);
    return e == hipSuccess ? QKPREP_OK : QKPREP_E_LAUNCH;
}

qkprep_status qkprep_mla_concat_rope_append(const qkprep_mla_params* p, hipStream_t stream) {
    if (!p) return QKPREP_E_NULL;
    if (p->struct_size != sizeof(qkprep_mla_params)) return QKPREP_E_VERSION;
    const int T = p->num_tokens;
    if (T < 0 || p->num_q_heads < 1 || p->nope_dim < 0) return QKPREP_E_SHAPE;
    if (p->rope_dim != 64) return QKPREP_E_UNSUPPORTED;
    if (p->kv_lora_rank <= 0 || p->kv_lora_rank % 512) return QKPREP_E_UNSUPPORTED;
    if (p->rope < 0 || p->rope > 1 || p->kv_dtype < 0 || p->kv_dtype > 1) return QKPREP_E_RANGE;
    if (p->block_size <= 0) return QKPREP_E_RANGE;
    if (p->q_mode < 0 || p->q_mode > 2) return QKPREP_E_RANGE;
    if (p->store_policy < 0 || p->store_policy > 1) return QKPREP_E_RANGE;
    const bool q8 = p->q_mode != QKPREP_Q_BF16;
    if (q8 && (p->nope_dim % 32 || p->nope_dim > 128)) return QKPREP_E_UNSUPPORTED;
    if (p->q_mode == QKPREP_Q_FP8_DYNAMIC) {
        if (p->num_q_heads > 128) return QKPREP_E_UNSUPPORTED;
        if (!(p->upper_max > 0.0f && p->upper_max <= 448.0f)) return QKPREP_E_RANGE;
    }
    if (T == 0) return QKPREP_OK;
    if (q8) {
        if (!p->q_out) return QKPREP_E_NULL;
        if (p->q_mode == QKPREP_Q_FP8_DYNAMIC && !p->q_scale) return QKPREP_E_NULL;
        if (p->q_mode == QKPREP_Q_FP8_STATIC && !p->q_scale_inv) return QKPREP_E_NULL;
        if (p->q_out_head_stride < p->nope_dim + p->rope_dim) return QKPREP_E_SHAPE;
        if (p->q_out_token_stride % 16 || p->q_out_head_stride % 16 || !aligned16(p->q_out))
            return QKPREP_E_ALIGN;
    }
    if (!p->q || !p->kv_c || !p->k_pe || !p->cos_sin_cache || !p->positions || !p->slot_mapping ||
        !p->kv_cache)
        return QKPREP_E_NULL;
    if (p->kv_dtype == QKPREP_FP8_E4M3 && !p->kv_scale) return QKPREP_E_NULL;
    const int row_len = p->kv_lora_rank + p->rope_dim;
    const int elt = p->kv_dtype == QKPREP_FP8_E4M3 ? 1 : 2;
    if (p->num_blocks < 1 || p->cos_sin_rows < 1) return QKPREP_E_SHAPE;
    if (p->q_head_stride < p->nope_dim + p->rope_dim) return QKPREP_E_SHAPE;
    if (p->kv_c_stride < p->kv_lora_rank || p->k_pe_stride < p->rope_dim) return QKPREP_E_SHAPE;
    if (p->block_stride < (int64_t)p->block_size * row_len) return QKPREP_E_SHAPE;
    if (p->nope_dim % 8 || p->q_head_stride % 8 || p->q_token_stride % 8 || p->kv_c_stride % 8 ||
        p->k_pe_stride % 8 || (p->block_stride * elt) % 16)
        return QKPREP_E_ALIGN;
    if (!aligned16(p->q) || !aligned16(p->kv_c) || !aligned16(p->k_pe) || !aligned16(p->cos_sin_cache) ||
        !aligned16(p->kv_cache))
        return QKPREP_E_ALIGN;

    MlaDevArgs a{};
    a.T = T; a.H = p->num_q_heads; a.nope_dim = p->nope_dim; a.kv_lora_rank = p->kv_lora_rank;
    a.q = static_cast<uint16_t*>(p->q);
    a.q_token_stride = p->q_token_stride; a.q_head_stride = p->q_head_stride;
    a.kv_c = static_cast<const uint16_t*>(p->kv_c); a.kv_c_stride = p->kv_c_stride;
    a.k_pe = static_cast<const uint16_t*>(p->k_pe); a.k_pe_stride = p->k_pe_stride;
    a.rope = p->rope;
    a.cos_sin = p->cos_sin_cache; a.cs_rows = p->cos_sin_rows;
    a.positions = p->positions; a.slot_mapping = p->slot_mapping;
    a.kv_cache = p->kv_cache;
    a.capacity = p->num_blocks * (int64_t)p->block_size;
    a.block_size = p->block_size; a.block_stride = p->block_stride;
    a.kv_scale = p->kv_scale;
    a.q_mode = p->q_mode;
    a.q_out = static_cast<uint8_t*>(p->q_out);
    a.q_out_token_stride = p->q_out_token_stride; a.q_out_head_stride = p->q_out_head_stride;
    a.q_scale = p->q_scale; a.q_scale_inv = p->q_scale_inv; a.upper_max = p->upper_max;
    a.nt_store = p->store_policy == QKPREP_STORE_KEEP ? 0 : 1;
    a.chunks_per_token = (a.H + 15) / 16 + 1;
    a.tokens_per_tile = kMaxTokensPerTile;
    a.total_items = (int64_t)T * a.chunks_per_token;
    if (a.total_items > INT32_MAX) return QKPREP_E_SHAPE;
    hipError_t e = q8 ? launch_mla_q8(a, p->kv_dtype, stream) : launch_mla_concat_rope(a, p->kv_dtype, stream);
    return e == hipSuccess ? QKPREP_OK : QKPREP_E_LAUNCH;
}

}  // extern "C"
