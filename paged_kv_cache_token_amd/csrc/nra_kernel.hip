// Fused Q/K RMSNorm + RoPE + (FP8) quantisation + paged KV append for gfx950.
//
// Operation: FlashInfer PR "fused QK RMSNorm + NeoX RoPE + FP8 E4M3 quantize +
// NHD paged-KV append" (Contract), TensorRT-LLM PR "Fuse Qwen3.5 gated QKV
// preprocessing" (Phase 2: Gemma norm + RoPE folded into the KV-append
// pass, strided rows), SGLang PR "fused Q/K RMSNorm + RoPE with
// cos_sin_cache" (fp32 table, int64 positions), vLLM issue "ROPE +
// KV-Cache-Write + pre-attn prepare-ops fusion" (model table: 64-dim heads,
// RoPE on part of the head with NoPE dims passed through).
//
// Mapping onto CDNA4 (one launch per call, 256-thread workgroups = 4 wave64):
//  * A head row of D bf16 elements is owned by G = D/16 lanes (4 for D=64,
//    8 for D=128, 16 for D=256).  Lane l of the group loads two 16-byte
//    vectors: elements [8l, 8l+8) and [R/2 + 8l, R/2 + 8l + 8) when l < R/16
//    (R rotated dims), else the 16 pass-through elements [16l, 16l+16).
//    Every NeoX pair (i, i + R/2) and every interleaved pair (2i, 2i+1) then
//    sits in one lane's registers: RoPE needs no lane exchange.  The common
//    R = D case is a separate instance with compile-time offsets, and R = 0
//    (no rotated dims) runs that layout with RoPE compiled out.  A wave
//    covers 64/G head rows of one token (a "chunk").
//  * The sum of squares and the FP8 amax are reduced over the G lanes of the
//    row only (DPP within the lane group), never across rows or tokens.
//  * Short calls give every workgroup a balanced, contiguous range of the
//    (token, chunk) items; long calls deal short spans of items round-robin,
//    so the resident workgroups stream through one narrow window of qkv at a
//    time.  Every
//    workgroup also owns a range of the requests; the grid is sized to what
//    stays resident.  Tiles of up to 16 tokens stage their cos/sin rows,
//    positions and cache row offsets in LDS; the norm weights are staged
//    once per workgroup.
//  * Loads are double-buffered and unconditional (rows past the run are
//    clamped to a valid row) so that the wait for one batch never drains the
//    loads of the next one.  Where one row's 128-byte line is split between
//    lanes (64-dim heads, partial rotary with 8 or 16 lanes per row), rows are
//    loaded one whole line per instruction and completed by a DPP mirror
//    exchange.
//  * All-or-nothing validation without a host sync or a second kernel:
//    every workgroup stages q_indptr / seq_lens in LDS, checks every request
//    and every page id the call will write, and reduces the verdict with one
//    barrier.  When every request writes at most two pages, each thread
//    checks its own request's pages; otherwise the pages are enumerated
//    through a prefix sum so that each thread checks about one.  Every
//    workgroup reads the same metadata, so all reach the same verdict.  An
//    invalid call makes the workgroups write -1 flags and nothing else.
//  * The latency chain of a small call is kept at two dependent memory
//    rounds: the first batch of qkv loads leaves at kernel entry, and the
//    page checks, row lookups, cos/sin rows and tail pages all issue in the
//    round after the request metadata arrives.
#include <type_traits>

#include "qkprep_device.h"
#include "qkprep_internal.h"

namespace qkprep {

namespace {

// Zeros that stand in for an input the call does not have (no tokens, no
// norm weights, slot addressing...): every prologue load then goes out
// unconditionally, with no lane mask or branch around it, which keeps the
// compiler's in-order load counters exact.  Never written.
__device__ __align__(16) const uint16_t g_zero_row[256] = {};

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
    // page ids are checked for the pages the call writes; K/V redirected to
    // out_k / out_v write no page, so none is read or checked
    if (a.redirect) return r;
    int lo_row = sl - ql;
    if (a.zero_tail && ql == 0 && sl > 0) lo_row = sl - 1;
    if (sl > lo_row) {
        r.first = fdiv31(lo_row, a.ps_div);
        r.count = fdiv31(sl - 1, a.ps_div) - r.first + 1;
    }
    return r;
}

// Validation, step 1: per-request checks and, on the full path, the
// block-wide exclusive prefix s_pre[0..B] of the number of pages each
// request writes, with the request and page-table column of each of the
// first kPageSlots pages (s_pgreq / s_pgcol).  With the page ids read as
// 16-byte vectors (a.pt_vec, at most kSearchRequests requests) it also writes
// s_vpre[0..B], the prefix of the number of whole vectors inside each
// request's written columns.  Needs s_indptr / s_seqlen staged.  Returns this thread's
// partial verdict and the path taken.
constexpr int kPageSlots = kBlockThreads;   // pages located by table lookup (one per thread)
static_assert(kSearchRequests <= 64, "the vector prefix is one wave's scan");

// The same pass also writes the request of each of the first tile's tokens
// (s_treq[t - t_first] for t in [t_first, t_first + ntok)), since it visits
// each request's q_indptr range anyway.
//
// Short path: with at most one request per thread and at most kFastPages
// pages per request (decodes, short prefills), each thread reads its own
// request's page ids right away, and the prefix and page slots are skipped
// (one barrier fewer; the page reads overlap the row lookups).  The choice
// is the same in every thread: a vote published by the pass's barrier.
constexpr int kFastPages = 2;

struct Verdict {
    int bad;        // this thread's partial verdict (page-id checks of the short path not yet applied)
    int fast;       // short path taken (uniform over the workgroup)
    int pg0, pg1;   // short path: the page ids of this thread's request
    int npg;        // short path: how many of pg0 / pg1 to check
};

__device__ Verdict validate_requests(const NraDevArgs& a, const int* s_indptr, const int* s_seqlen, int* s_pre,
                                     int* s_wave, int* s_vote, int* s_pgreq, int* s_pgcol, int* s_vpre,
                                     int* s_treq, int t_first, int ntok) {
    const int tid = threadIdx.x;
    const int B = a.B;
    int bad = 0;
    if (tid == 0 && (s_indptr[0] != 0 || s_indptr[B] != a.T)) bad = 1;
    const int per = (B + kBlockThreads - 1) / kBlockThreads;
    const int lo = min(B, tid * per), hi = min(B, lo + per);
    int sum = 0, few = 1, vsum = 0;
    ReqPages rp_lo{0, 0, 0};   // request lo's pages, kept for the second pass
    for (int b = lo; b < hi; ++b) {
        const int t0 = max(s_indptr[b], t_first), t1 = min(s_indptr[b + 1], t_first + ntok);
        for (int t = t0; t < t1; ++t) s_treq[t - t_first] = b;
        ReqPages rp = request_pages(a, s_indptr, s_seqlen, b);
        if (b == lo) rp_lo = rp;
        bad |= rp.bad;
        sum += rp.count;
        few &= rp.count <= kFastPages ? 1 : 0;
        // whole 16-byte vectors of the page-table row inside columns [first, first + count)
        if (rp.count > 0) vsum += max(((rp.first + rp.count) >> 2) - ((rp.first + 3) >> 2), 0);
    }
    // the own request's page ids (a valid request's pages lie inside its
    // page-table row; an invalid one has count 0 and reads the zero row)
    const int own = (per == 1 && lo < hi) ? rp_lo.count : 0;
    const int* zi = reinterpret_cast<const int*>(g_zero_row);
    const int* q0 = own >= 1 ? a.page_table + (int64_t)lo * a.maxp + rp_lo.first : zi;
    const int pg0 = gld(q0);
    const int pg1 = gld(own >= 2 ? q0 + 1 : zi);
    const int lane = tid & 63, wave = tid >> 6;
    const int incl = wave_inclusive_scan(sum);
    if (lane == 63) s_wave[wave] = incl;
    const bool wave_few = __ballot(few == 0) == 0;
    if (lane == 0) s_vote[wave] = wave_few ? 1 : 0;
    __syncthreads();
    if (per == 1 && (s_vote[0] & s_vote[1] & s_vote[2] & s_vote[3]))
        return Verdict{bad, 1, pg0, pg1, own};
    int base = 0;
    for (int w = 0; w < wave; ++w) base += s_wave[w];
    int run = base + incl - sum;
    for (int b = lo; b < hi; ++b) {
        s_pre[b] = run;
        const ReqPages rp = b == lo ? rp_lo : request_pages(a, s_indptr, s_seqlen, b);
        // the first kPageSlots pages of the call: their request and column
        // (many requests: each writes its few slots; few requests find their
        // pages by binary search instead, see page_id_ptr)
        for (int k = run; a.B > kSearchRequests && k < min(run + rp.count, kPageSlots); ++k) {
            s_pgreq[k] = b;
            s_pgcol[k] = rp.first + (k - run);
        }
        run += rp.count;
    }
    if (tid == kBlockThreads - 1) s_pre[B] = base + incl;
    if (a.pt_vec) {
        // B <= kSearchRequests <= 64: every request is owned by a lane of wave 0
        const int vincl = wave_inclusive_scan(vsum);
        if (wave == 0 && lo < hi) s_vpre[lo] = vincl - vsum;
        if (tid == B - 1) s_vpre[B] = vincl;
    }
    __syncthreads();
    return Verdict{bad, 0, 0, 0, 0};
}

// Validation, step 2: every page id the call writes must lie in the pool.
// Thread k checks pages k, k + 256, ... of the call's flattened page list;
// page_id_ptr() is the address of page k (the first round's check).
__device__ __forceinline__ const int* page_id_ptr(const NraDevArgs& a, const int* s_indptr, const int* s_seqlen,
                                                  const int* s_pre, int k) {
    const int b = lds_upper_bound(s_pre, a.B + 1, k) - 1;
    const ReqPages rp = request_pages(a, s_indptr, s_seqlen, b);
    return a.page_table + (int64_t)b * a.maxp + rp.first + (k - s_pre[b]);
}

__device__ __forceinline__ int page_out_of_pool(const NraDevArgs& a, int p) {
    return (p < 0 || p >= a.num_pages) ? 1 : 0;
}

// Pages k = k0, k0 + 256, ... (< total) of the flattened list: the request
// of each page is found by walking forward from the request of k0 (one
// binary search per thread), and the page ids are loaded kPageBatch at a
// time with independent loads, so a call that writes many pages (a long
// prefill at a small page size) costs a few memory round trips per
// workgroup instead of one per 256 pages.  Returns 1 if any id is outside
// the pool.
constexpr int kPageBatch = 16;

__device__ int pages_out_of_pool(const NraDevArgs& a, const int* s_indptr, const int* s_seqlen, const int* s_pre,
                                 int k0, int total) {
    if (k0 >= total) return 0;
    int b = lds_upper_bound(s_pre, a.B + 1, k0) - 1;
    ReqPages rp = request_pages(a, s_indptr, s_seqlen, b);
    int bad = 0;
    for (int kb = k0; kb < total; kb += kBlockThreads * kPageBatch) {
        int v[kPageBatch];
#pragma unroll
        for (int u = 0; u < kPageBatch; ++u) {
            const int k = kb + u * kBlockThreads;
            const bool in = k < total;
            // (requests that write no page have s_pre[b] == s_pre[b + 1])
            while (in && k >= s_pre[b + 1]) {
                ++b;
                rp = request_pages(a, s_indptr, s_seqlen, b);
            }
            v[u] = gld(in ? a.page_table + (int64_t)b * a.maxp + rp.first + (k - s_pre[b])
                          : reinterpret_cast<const int*>(g_zero_row));
        }
#pragma unroll
        for (int u = 0; u < kPageBatch; ++u) bad |= page_out_of_pool(a, v[u]);
    }
    return bad;
}


// Every page id the call writes, with the page table read as 16-byte
// vectors (a.pt_vec: the table and its rows are 16-byte aligned).  Each
// request's written columns [first, first + count) split into whole vectors
// and at most 3 + 3 columns at the two ends.  The whole vectors of all
// requests are numbered consecutively (prefix s_vpre); thread k takes
// vectors k, k + 256, ..., kVecBatch of them in flight, walking forward over
// the requests as the pages walk does, and keeps the unsigned maximum of the
// ids (a negative id compares above the pool as well).  Thread b < B reads
// the end columns of request b one by one, in the same round as its first
// vectors.  Returns 1 if any id is outside the pool.
constexpr int kVecBatch = 4;

__device__ __forceinline__ int first_whole_vector(int first) { return (first + 3) >> 2; }

__device__ int page_vectors_out_of_pool(const NraDevArgs& a, const int* s_indptr, const int* s_seqlen,
                                        const int* s_vpre) {
    const int tid = threadIdx.x;
    const int* zi = reinterpret_cast<const int*>(g_zero_row);
    // the end columns of request tid, outside its whole vectors (a column
    // not written reads the zero row, which is inside the pool)
    uint32_t e[6];
    {
        const int b = min(tid, a.B - 1);
        const ReqPages rp = request_pages(a, s_indptr, s_seqlen, b);
        const bool own = tid < a.B && rp.count > 0;
        const int lo = rp.first, hi = rp.first + rp.count;
        const int head_end = min(hi, 4 * first_whole_vector(lo));   // [lo, head_end)
        const int tail_beg = max(lo, 4 * (hi >> 2));                // [tail_beg, hi)
        const int* rowp = a.page_table + (int64_t)b * a.maxp;
#pragma unroll
        for (int j = 0; j < 3; ++j) {
            e[j] = (uint32_t)gld(own && lo + j < head_end ? rowp + lo + j : zi);
            e[3 + j] = (uint32_t)gld(own && tail_beg + j < hi ? rowp + tail_beg + j : zi);
        }
    }
    // the whole vectors
    uint32_t mx = 0;
    const int total = s_vpre[a.B];
    if (tid < total) {
        int b = lds_upper_bound(s_vpre, a.B + 1, tid) - 1;
        int v_lo = s_vpre[b], v_hi = s_vpre[b + 1];
        const u32x4_t* row = reinterpret_cast<const u32x4_t*>(a.page_table + (int64_t)b * a.maxp) +
                             first_whole_vector(request_pages(a, s_indptr, s_seqlen, b).first);
        for (int kb = tid; kb < total; kb += kBlockThreads * kVecBatch) {
            u32x4_t v[kVecBatch];
#pragma unroll
            for (int u = 0; u < kVecBatch; ++u) {
                const int k = kb + u * kBlockThreads;
                const bool in = k < total;
                // (requests with no whole vector have s_vpre[b] == s_vpre[b + 1])
                while (in && k >= v_hi) {
                    ++b;
                    v_lo = v_hi;
                    v_hi = s_vpre[b + 1];
                    row = reinterpret_cast<const u32x4_t*>(a.page_table + (int64_t)b * a.maxp) +
                          first_whole_vector(request_pages(a, s_indptr, s_seqlen, b).first);
                }
                v[u] = gld(in ? row + (k - v_lo) : reinterpret_cast<const u32x4_t*>(g_zero_row));
            }
#pragma unroll
            for (int u = 0; u < kVecBatch; ++u) mx = max(max(mx, max(v[u].x, v[u].y)), max(v[u].z, v[u].w));
        }
    }
#pragma unroll
    for (int j = 0; j < 6; ++j) mx = max(mx, e[j]);
    return mx >= (uint32_t)a.num_pages ? 1 : 0;
}


template <int D, int QMODE, bool KVFP8>
struct KvType {
    typedef typename std::conditional<KVFP8, uint8_t, uint16_t>::type type;
};

// Which two 8-element pieces of a head row lane gl of its group holds.
// With R rotated dims (R a multiple of 16), lanes gl < R/16 ("rope lanes")
// hold [8 gl, 8 gl + 8) and [R/2 + 8 gl, R/2 + 8 gl + 8): every NeoX pair
// (i, i + R/2) and every interleaved pair (2i, 2i+1) then sits in one
// lane's registers.  The other lanes hold 16 pass-through dims
// [16 gl, 16 gl + 16).  For R = D this is the split [8 gl, ..) | [D/2 + 8 gl, ..).
struct LaneMap {
    int o0, o1;      // element offsets of the two vectors in the head row
    int hr, qr;      // R/2 and R/4: offsets of the sine half and of the second vector's angles
    int fp8_store;   // 0: one 16-byte store; 1: swap a half with the neighbour lane; 2: two 8-byte stores
    bool rope;
};

// Rotary layouts, one kernel instance each: the whole head rotates (R = D),
// its first R dims do (0 < R < D), or none do (R = 0; the whole-head layout,
// which only has to be the same for loads and stores, with RoPE compiled out)
enum : int { kRotWhole = 0, kRotPart = 1, kRotNone = 2 };

template <int D, int ROT>
__device__ __forceinline__ LaneMap lane_map(int rot, int gl) {
    LaneMap m;
    if constexpr (ROT != kRotPart) {
        // compile-time split, immediate store offsets
        m.rope = ROT == kRotWhole;
        m.o0 = 8 * gl;
        m.o1 = D / 2 + 8 * gl;
        m.hr = D / 2;
        m.qr = D / 4;
        m.fp8_store = 1;
        return m;
    }
    m.rope = gl < (rot >> 4);
    m.hr = rot >> 1;
    m.qr = rot >> 2;
    m.o0 = m.rope ? 8 * gl : 16 * gl;
    m.o1 = m.rope ? (rot >> 1) + 8 * gl : 16 * gl + 8;
    // rope lanes pair up (and the swapped 16 bytes stay 16-byte aligned)
    // when R/2 is a multiple of 16
    m.fp8_store = !m.rope ? 0 : ((rot & 31) == 0 ? 1 : 2);
    return m;
}

// E4M3 codes of the lane's two pieces (lo at o0, hi at o1) into a head row
// of bytes.  Paired rope lanes trade one 8-byte half so that each writes 16
// contiguous bytes: the even lane [o0, o0 + 16), the odd lane [o1 - 8, o1 + 8).
template <bool NT>
__device__ __forceinline__ void store_fp8_lane(uint8_t* row, int gl, const LaneMap& m, uint2 lo, uint2 hi) {
    const bool odd = gl & 1;
    const uint2 send = odd ? lo : hi;
    uint2 recv;
    recv.x = (uint32_t)__builtin_amdgcn_update_dpp(0, (int)send.x, kDppQuadSwap1, 0xF, 0xF, false);
    recv.y = (uint32_t)__builtin_amdgcn_update_dpp(0, (int)send.y, kDppQuadSwap1, 0xF, 0xF, false);
    if (m.fp8_store != 2) {
        // paired rope lanes and pass-through lanes in one store instruction,
        // so a row's 128-byte lines are written by a single instruction
        const bool swap = m.fp8_store == 1;
        const uint4 v = !swap ? make_uint4(lo.x, lo.y, hi.x, hi.y)
                        : odd ? make_uint4(recv.x, recv.y, hi.x, hi.y) : make_uint4(lo.x, lo.y, recv.x, recv.y);
        st16p<NT>(row + ((swap && odd) ? m.o1 - 8 : m.o0), v);
    } else {
        st8p<NT>(row + m.o0, lo);
        st8p<NT>(row + m.o1, hi);
    }
}

// max over aligned groups of n lanes (n = 1, 2, 4, 8 or 16, the same for
// the whole wave); every lane of a group receives the group's max
// (non-negative values: the reduction runs on their bit patterns)
__device__ __forceinline__ float subgroup_max(float v, int n) {
    uint32_t u = __float_as_uint(v);
    if (n >= 2) u = max(u, dpp_u<kDppQuadSwap1>(u));
    if (n >= 4) u = max(u, dpp_u<kDppQuadSwap2>(u));
    if (n >= 8) u = max(u, dpp_u<kDppRowHalfMirror>(u));
    if (n >= 16) u = max(u, dpp_u<kDppRowMirror>(u));
    return __uint_as_float(u);
}

// E4M3 codes of a K or V head row with dynamic scales: one per group of
// a.kv_group dims, s = max(amax, 1e-6) / 448, stored at sc[group].  The row
// is f * x (f > 0: the RMSNorm factor not yet applied to x, or 1), so the
// amax is f * max|x| and the payload multiplier f / s.  With a.kv_group == D
// the whole row shares one scale; smaller groups lie inside one half of the
// lane split (whole-head rotary layout: the lane holds dims [8 gl, 8 gl + 8)
// and [D/2 + 8 gl, D/2 + 8 gl + 8)) and span g/8 lanes.
template <int D>
__device__ __forceinline__ void kv_fp8_dynamic(const NraDevArgs& a, int gl, const float* x, float f, float* sc,
                                               uint2& lo, uint2& hi) {
    constexpr int G = D / 16;
    constexpr float kInv448 = 1.0f / 448.0f;
    float m0 = 0.0f, m1 = 0.0f;
#pragma unroll
    for (int i = 0; i < 8; ++i) {
        m0 = __builtin_fmaxf(m0, __builtin_fabsf(x[i]));
        m1 = __builtin_fmaxf(m1, __builtin_fabsf(x[8 + i]));
    }
    if (a.kv_group == D) {
        const float s = max_nonneg(group_max<G>(max_nonneg(m0, m1)) * f, 1e-6f) * kInv448;
        const float mul = f * __builtin_amdgcn_rcpf(s);
        if (gl == 0) sc[0] = s;
        lo = pack8_fp8_bounded(x, mul);
        hi = pack8_fp8_bounded(x + 8, mul);
    } else {
        const int n = a.kv_group >> 3;
        const float s0 = max_nonneg(subgroup_max(m0, n) * f, 1e-6f) * kInv448;
        const float s1 = max_nonneg(subgroup_max(m1, n) * f, 1e-6f) * kInv448;
        if ((gl & (n - 1)) == 0) {
            sc[(8 * gl) / a.kv_group] = s0;
            sc[(D / 2 + 8 * gl) / a.kv_group] = s1;
        }
        lo = pack8_fp8_bounded(x, f * __builtin_amdgcn_rcpf(s0));
        hi = pack8_fp8_bounded(x + 8, f * __builtin_amdgcn_rcpf(s1));
    }
}

// Encodes and stores head row r of tile token ti (global token t) whose two
// 16-byte vectors v0 / v1 (elements at lm.o0 / lm.o1) are in registers.
// Q/K rows: RMSNorm (weights from LDS), RoPE on the rotated dims (cos/sin
// row from LDS), then bf16 / E4M3.  V rows: copy or E4M3.  `k` holds the
// per-call constants.
struct RowConsts {
    float inv_k, inv_v, q_static, inv_um;
    int qs_hstride;
    int kv_ng;       // dynamic K/V scales per head row (0: static scalars)
    float* s_qs;     // non-null: stage dynamic Q scales in LDS [token][head]
};

template <int D, int QMODE, bool KVFP8, bool NT>
__device__ __forceinline__ void process_row(const NraDevArgs& a, int t, int ti, int r, int gl, const LaneMap& lm,
                                            uint4 v0, uint4 v1, const float* s_w, const float* s_cs_row,
                                            const int64_t* s_koff, const int64_t* s_voff, const int64_t* s_qsoff,
                                            const int64_t* s_srow, const RowConsts& k) {
    constexpr int G = D / 16;
    typedef typename KvType<D, QMODE, KVFP8>::type kv_t;
    // Cache rows (a few hundred bytes to 1 KiB per token into pages) take
    // ordinary stores whatever the policy: merged in L2 and written back, they
    // cost less than streaming stores (16k-token FP8 prefill 94.5 -> 91.4 us,
    // the T = 14 876 draw 87.0 -> 84.1 us, rotating buffers), while the long
    // contiguous Q rows stream when the policy says so.
    constexpr bool NTKV = false;
    if (r >= a.Hq + a.Hkv) {
        // V head: raw copy (bf16 cache) or x / v_scale (FP8 cache)
        const int64_t voff = s_voff[ti];
        if (voff < 0) return;
        const int vh = r - a.Hq - a.Hkv;
        kv_t* row = reinterpret_cast<kv_t*>(a.v_cache) + voff + vh * D;
        if constexpr (KVFP8) {
            float x[16];
            unpack8(v0, x);
            unpack8(v1, x + 8);
            uint2 lo, hi;
            if (k.kv_ng) {
                kv_fp8_dynamic<D>(a, gl, x, 1.0f, a.v_scale_out + (s_srow[ti] * a.Hkv + vh) * k.kv_ng, lo, hi);
            } else {
                lo = pack8_fp8(x, k.inv_v);
                hi = pack8_fp8(x + 8, k.inv_v);
            }
            store_fp8_lane<NTKV>(reinterpret_cast<uint8_t*>(row), gl, lm, lo, hi);
        } else {
            st16p<NTKV>(row + lm.o0, v0);
            st16p<NTKV>(row + lm.o1, v1);
        }
        return;
    }
    const bool is_q = r < a.Hq;
    float x[16];
    unpack8(v0, x);
    unpack8(v1, x + 8);
    // RMSNorm factor not yet applied to x.  Rows that end as E4M3 (and
    // write no bf16 copy) apply it with their payload multiplier, after
    // RoPE (which is linear): one multiply per element fewer.  bf16 rows
    // apply it here.
    float f = 1.0f;
    if (a.norm != 0) {
        float ss = sumsq8_bf16(v1, sumsq8_bf16(v0, 0.0f));
        ss = group_sum<G>(ss);
        // the argument is >= eps > 0; the floor keeps v_rsq off denormal
        // inputs (an all-zero row with eps < 2^-126 stays zero)
        const float inv = __builtin_amdgcn_rsqf(__builtin_fmaxf(fmaf(ss, 1.0f / (float)D, a.eps), 1.17549435e-38f));
        const float* w = s_w + (is_q ? 0 : D);
        const float4 w0 = *reinterpret_cast<const float4*>(w + lm.o0);
        const float4 w1 = *reinterpret_cast<const float4*>(w + lm.o0 + 4);
        const float4 w2 = *reinterpret_cast<const float4*>(w + lm.o1);
        const float4 w3 = *reinterpret_cast<const float4*>(w + lm.o1 + 4);
        const float wv[16] = {w0.x, w0.y, w0.z, w0.w, w1.x, w1.y, w1.z, w1.w,
                              w2.x, w2.y, w2.z, w2.w, w3.x, w3.y, w3.z, w3.w};
        const bool late = is_q ? QMODE != 0 : (KVFP8 && a.k_out == nullptr);
        if (late) {
            f = inv;
#pragma unroll
            for (int i = 0; i < 16; ++i) x[i] = x[i] * wv[i];
        } else {
#pragma unroll
            for (int i = 0; i < 16; ++i) x[i] = x[i] * inv * wv[i];
        }
    }
    if (lm.rope) {
        const int hr = lm.hr;
        if (a.rope == 0) {
            // NeoX: pair i of the lane = dims (8 gl + i, R/2 + 8 gl + i), angle 8 gl + i
            const float4 c0 = *reinterpret_cast<const float4*>(s_cs_row + 8 * gl);
            const float4 c1 = *reinterpret_cast<const float4*>(s_cs_row + 8 * gl + 4);
            const float4 s0 = *reinterpret_cast<const float4*>(s_cs_row + hr + 8 * gl);
            const float4 s1 = *reinterpret_cast<const float4*>(s_cs_row + hr + 8 * gl + 4);
            const float c[8] = {c0.x, c0.y, c0.z, c0.w, c1.x, c1.y, c1.z, c1.w};
            const float s[8] = {s0.x, s0.y, s0.z, s0.w, s1.x, s1.y, s1.z, s1.w};
#pragma unroll
            for (int i = 0; i < 8; ++i) {
                const float xa = x[i], xb = x[8 + i];
                x[i] = xa * c[i] - xb * s[i];
                x[8 + i] = xb * c[i] + xa * s[i];
            }
        } else {
            // interleaved: the first vector holds angles 4 gl .. 4 gl + 3, the
            // second R/4 + 4 gl .. R/4 + 4 gl + 3
            const int qr = lm.qr;
            const float4 c0 = *reinterpret_cast<const float4*>(s_cs_row + 4 * gl);
            const float4 c1 = *reinterpret_cast<const float4*>(s_cs_row + qr + 4 * gl);
            const float4 s0 = *reinterpret_cast<const float4*>(s_cs_row + hr + 4 * gl);
            const float4 s1 = *reinterpret_cast<const float4*>(s_cs_row + hr + qr + 4 * gl);
            const float c[8] = {c0.x, c0.y, c0.z, c0.w, c1.x, c1.y, c1.z, c1.w};
            const float s[8] = {s0.x, s0.y, s0.z, s0.w, s1.x, s1.y, s1.z, s1.w};
#pragma unroll
            for (int m = 0; m < 8; ++m) {
                const int i0 = (m < 4) ? 2 * m : 8 + 2 * (m - 4);
                const float xa = x[i0], xb = x[i0 + 1];
                x[i0] = xa * c[m] - xb * s[m];
                x[i0 + 1] = xb * c[m] + xa * s[m];
            }
        }
    }
    if (is_q) {
        const int h = r;
        if constexpr (QMODE == 0) {
            uint16_t* row = reinterpret_cast<uint16_t*>(a.q_out) + (int64_t)t * a.q_out_stride + h * D;
            st16p<NT>(row + lm.o0, pack8_bf16(x));
            st16p<NT>(row + lm.o1, pack8_bf16(x + 8));
        } else {
            uint8_t* row = reinterpret_cast<uint8_t*>(a.q_out) + (int64_t)t * a.q_out_stride + h * D;
            if constexpr (QMODE == 1) {
                // the row is f * x: amax = f * max|x|, s = max(amax, 1e-6) /
                // upper_max, payload = x * (f / s)
                float amax = 0.0f;
#pragma unroll
                for (int i = 0; i < 16; ++i) amax = __builtin_fmaxf(amax, __builtin_fabsf(x[i]));
                amax = group_max<G>(amax) * f;
                const float sc = max_nonneg(amax, 1e-6f) * k.inv_um;
                const float mul = f * __builtin_amdgcn_rcpf(sc);
                if (gl == 0) {
                    if (k.s_qs) k.s_qs[ti * a.Hq + h] = sc;
                    else a.q_scale[s_qsoff[ti] + (int64_t)h * k.qs_hstride] = sc;
                }
                store_fp8_lane<NT>(row, gl, lm, pack8_fp8_bounded(x, mul), pack8_fp8_bounded(x + 8, mul));
            } else {
                const float mul = f * k.q_static;
                store_fp8_lane<NT>(row, gl, lm, pack8_fp8(x, mul), pack8_fp8(x + 8, mul));
            }
        }
    } else {
        const int kh = r - a.Hq;
        const int64_t koff = s_koff[ti];
        if (koff >= 0) {
            kv_t* row = reinterpret_cast<kv_t*>(a.k_cache) + koff + kh * D;
            if constexpr (KVFP8) {
                uint2 lo, hi;
                if (k.kv_ng) {
                    kv_fp8_dynamic<D>(a, gl, x, f, a.k_scale_out + (s_srow[ti] * a.Hkv + kh) * k.kv_ng, lo, hi);
                } else {
                    lo = pack8_fp8(x, f * k.inv_k);
                    hi = pack8_fp8(x + 8, f * k.inv_k);
                }
                store_fp8_lane<NTKV>(reinterpret_cast<uint8_t*>(row), gl, lm, lo, hi);
            } else {
                st16p<NTKV>(row + lm.o0, pack8_bf16(x));
                st16p<NTKV>(row + lm.o1, pack8_bf16(x + 8));
            }
        }
        if (a.k_out) {
            uint16_t* ko = a.k_out + (int64_t)t * a.k_out_stride + kh * D;
            st16p<NT>(ko + lm.o0, pack8_bf16(x));
            st16p<NT>(ko + lm.o1, pack8_bf16(x + 8));
        }
    }
}

// (token, chunk) cursor over a wave's run of items; chunk c of token t
// covers head rows [c * RPW, c * RPW + RPW).
struct Cursor {
    int t, c, left;
    __device__ __forceinline__ void advance(int cpt) {
        const bool wrap = c + 1 == cpt;
        c = wrap ? 0 : c + 1;
        t += wrap ? 1 : 0;
        --left;
    }
};

template <int D, int QMODE, bool KVFP8, int ROT, int MEM, bool TL>
__global__ __launch_bounds__(kBlockThreads) __attribute__((amdgpu_waves_per_eu(4))) void nra_kernel(const NraDevArgs a) {
    constexpr bool PART = ROT == kRotPart;
    constexpr bool NTL = MEM != kMemInPlace;     // qkv read once: streaming loads
    constexpr bool NTS = MEM == kMemStream;      // Q rows: streaming stores (K/V rows: ordinary)
    constexpr int G = D / 16;        // lanes per head row
    constexpr int RPW = 64 / G;      // head rows per wave
    constexpr int U = kBatch;
    constexpr int D4 = D / 4;        // float4 per cos/sin row
    // 64-dim heads: four lanes hold a 128-byte row, so one load per
    // lane-vector would read only half of each row's line per instruction
    // (measured ~10 % slower for streaming loads); rows are read in pairs of
    // whole lines instead, in every rotary layout
    constexpr bool kPairRows = D == 64;
    // Rotary over at most half the head (8 or 16 lanes per row): lanes
    // 0 .. G/2-1 then hold exactly the first half of the row, but the rope
    // lanes' two vectors lie R/2 apart, so one load instruction would touch
    // both lines of a row partly; each lane instead loads its first-half
    // vector and its mirror partner's (or the partner's and its own
    // second-half one), and a mirror exchange hands every lane its own
    const bool half_rot = PART && D >= 128 && 2 * a.rot <= D;
    // Rotary over more than half the head: with P = G - R/16 pass-through
    // lanes, the P lowest lanes (rope lanes) and the P highest (pass lanes)
    // hold the two lines' leftover vectors of each other, so they load for
    // their mirror partner and trade; the rope lanes in between load their
    // own two vectors
    const bool wide_rot = PART && D >= 128 && 2 * a.rot > D;
    typedef typename KvType<D, QMODE, KVFP8>::type kv_t;

    // q_indptr [B+1] | seq_lens [B] | page prefix [B+1] | (padded q_scale) staged scales [TPB][Hq]
    extern __shared__ int s_dyn[];
    __shared__ int s_wave[4];
    __shared__ int s_vote[4];
    __shared__ __align__(16) float s_w[2 * D];                       // q | k norm weights
    __shared__ __align__(16) float s_cs[kMaxTokensPerTile * D];      // cos/sin rows of the tile
    __shared__ int s_pos[kMaxTokensPerTile];
    __shared__ int64_t s_koff[kMaxTokensPerTile];
    __shared__ int64_t s_voff[kMaxTokensPerTile];
    __shared__ int64_t s_qsoff[kMaxTokensPerTile];
    __shared__ int64_t s_srow[kMaxTokensPerTile];    // cache row (page * page_size + row) or token, for K/V scales
    __shared__ int s_tail[kTailPrefetch];
    __shared__ int s_pgreq[kPageSlots];              // request of page slot k
    __shared__ int s_pgcol[kPageSlots];              // its page-table column
    __shared__ int s_vpre[kSearchRequests + 1];      // page-id vectors before request b (a.pt_vec)
    __shared__ int s_treq[kMaxTokensPerTile];        // request of each tile token
    __shared__ int s_flag[4];

    {
        // One scalar load per 32 bytes of the arguments at entry brings every
        // line of the struct into the scalar cache in one burst (on a fresh
        // launch the kernarg loads miss), and the later loads of the other
        // fields hit there.  Forcing all ~90 dwords into SGPRs instead kept
        // them live: the allocator then spilled ~180 SGPRs into VGPR lanes,
        // and the readlanes cost 0.2-0.6 us per decode and ~1 % of a long
        // prefill.
        const uint32_t* w = reinterpret_cast<const uint32_t*>(&a);
#pragma unroll
        for (int i = 0; i < (int)(sizeof(NraDevArgs) / 4); i += 8) asm volatile("" ::"s"(w[i]));
    }
    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);   // wave-uniform: cursor math stays scalar
    const int grp = lane / G;        // head-row slot of this lane in the wave
    const int gl = lane % G;         // lane inside the head row
    const LaneMap lm = lane_map<D, ROT>(a.rot, gl);
    int ld_o0 = lm.o0, ld_o1 = lm.o1;   // element offsets this lane loads
    if constexpr (kPairRows) {
        // rows 2p and 2p+1: a lane of row 2p loads its own first vector and
        // the first vector of its mirror partner in row 2p+1 (lane G-1-gl
        // there); a lane of row 2p+1 loads its partner's second vector in
        // row 2p and its own second vector
        const LaneMap pm = lane_map<D, ROT>(a.rot, G - 1 - gl);
        const bool even = (grp & 1) == 0;
        ld_o0 = even ? lm.o0 : pm.o1;
        ld_o1 = even ? pm.o0 : lm.o1;
    }
    bool xlo = false, xhi = false;       // lane trades its second / first vector
    if constexpr (PART && D >= 128) {
        const LaneMap pm = lane_map<D, ROT>(a.rot, G - 1 - gl);
        const int P = half_rot ? G / 2 : G - (a.rot >> 4);
        xlo = gl < P;
        xhi = gl >= G - P;
        if (xlo) {
            ld_o0 = lm.o0;
            ld_o1 = pm.o0;
        } else if (xhi) {
            ld_o0 = pm.o1;
            ld_o1 = lm.o1;
        }
    }
    int* s_indptr = s_dyn;
    int* s_seqlen = s_dyn + (a.B + 1);
    int* s_pre = s_dyn + (2 * a.B + 1);

    const int CPT = a.chunks_per_token;
    const int TPB = a.tokens_per_tile;
    const int64_t row_elems = (int64_t)a.Hkv * D;
    // Item ranges of this workgroup: one balanced contiguous range, or (when
    // a.interleave > 0) spans of a.interleave items dealt round-robin, so that
    // the workgroups running at any moment read neighbouring parts of qkv.
    int range_k = 0, blo = 0, bhi = 0;
    auto next_range = [&]() -> bool {
        if (a.interleave == 0) {
            if (range_k++ > 0) return false;
            // total * b / grid = items_q * b + items_r * b / grid (items_r * b < grid^2)
            const int b = blockIdx.x;
            blo = a.items_q * b + fdiv31(a.items_r * b, a.grid_div);
            bhi = a.items_q * (b + 1) + fdiv31(a.items_r * (b + 1), a.grid_div);
            return blo < bhi;
        }
        const int64_t span = a.interleave;
        // Workgroup b takes span sidx(b) of every round, a permutation of
        // [0, grid) under which runs of kXcdRun consecutive spans land on one
        // XCD (the dispatcher deals workgroups to the kXcds XCDs round-robin
        // by index): the padded Q-scale pieces
        // of neighbouring spans then meet in one L2 and leave it as whole
        // lines, while the round still covers the same narrow window of qkv.
        // (Identity when the grid is not a multiple of kXcds * kXcdRun.)
        int64_t sidx = blockIdx.x;
        if (a.grid % (kXcds * kXcdRun) == 0) {
            const int b = blockIdx.x, xcd = b % kXcds, slot = b / kXcds;
            sidx = (int64_t)(slot / kXcdRun) * (kXcds * kXcdRun) + xcd * kXcdRun + slot % kXcdRun;
        }
        const int64_t tile = sidx + (int64_t)(range_k++) * a.grid;
        if (tile * span >= a.total_items) return false;
        blo = (int)(tile * span);
        bhi = (int)min((int64_t)a.total_items, tile * span + span);
        return true;
    };

    uint4 bufA[U][2], bufB[U][2];
    Cursor ld{0, 0, 0}, pr{0, 0, 0};
    int sub_lo = 0, t_first = 0, ntok = 0, sub_hi = 0;
    // Loads of the next U head rows of the wave's run (no metadata needed).
    // Always exactly 2 U loads: the compiler's wait counters then stay exact,
    // and a wait for one batch never has to drain the batch issued after it.
    // Rows past the run or past R read the 512-byte zero row instead, a line
    // that stays in the caches: a clamped qkv row there made the last batch of each
    // tile (and of each wave) wait for a memory round trip of its own (B=256
    // decode 9.4 -> 8.7 us, the 16k prefill 95.6 -> 94.7 us).
    auto load_batch = [&](uint4 (&buf)[U][2]) {
#pragma unroll
        for (int u = 0; u < U; ++u) {
            const int tt = ld.left > 0 ? ld.t : t_first;
            const uint16_t* tok = (a.T > 0 ? a.qkv : g_zero_row) + (int64_t)tt * a.qkv_stride;
            if constexpr (kPairRows) {
                // rows 2p and 2p+1 of the chunk: the first load reads the whole
                // line of row 2p (its lanes their first vectors, row 2p+1's
                // lanes its second vectors, mirrored), the second the whole
                // line of row 2p+1; pair_exchange then gives every lane its own
                const int ra = ld.c * RPW + (grp & ~1), rb = ra + 1;
                const uint16_t* sa = (ld.left > 0 && ra < a.R) ? tok + ra * D + ld_o0 : g_zero_row + ld_o0;
                const uint16_t* sb = (ld.left > 0 && rb < a.R) ? tok + rb * D + ld_o1 : g_zero_row + ld_o1;
                if constexpr (NTL) {
                    buf[u][0] = ld16_stream(sa);
                    buf[u][1] = ld16_stream(sb);
                } else {
                    buf[u][0] = ld16(sa);
                    buf[u][1] = ld16(sb);
                }
                ld.advance(CPT);
                continue;
            }
            const int r = ld.c * RPW + grp;
            const bool ok = ld.left > 0 && r < a.R;
            const uint16_t* src = ok ? tok + r * D : g_zero_row;
            if constexpr (NTL) {
                buf[u][0] = ld16_stream(src + ld_o0);
                buf[u][1] = ld16_stream(src + ld_o1);
            } else {
                buf[u][0] = ld16(src + ld_o0);
                buf[u][1] = ld16(src + ld_o1);
            }
            ld.advance(CPT);
        }
    };
    // tile bounds and this wave's run inside it
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
    // request of every tile token, written by the threads that own the
    // requests (each request covers one run of tokens); made visible by the
    // next barrier.  Malformed metadata can leave entries unset: readers
    // clamp, and the verdict rejects the call.
    auto scatter_tokens = [&]() {
        const int per = (a.B + kBlockThreads - 1) / kBlockThreads;
        const int lo = min(a.B, tid * per), hi = min(a.B, lo + per);
        for (int b = lo; b < hi; ++b) {
            const int t0 = max(s_indptr[b], t_first), t1 = min(s_indptr[b + 1], t_first + ntok);
            for (int t = t0; t < t1; ++t) s_treq[t - t_first] = b;
        }
    };
    // per-token metadata that needs no request lookup (position, slot):
    // fetched into registers, then written to LDS
    struct TokMeta {
        int64_t pos, slot;
    };
    // (every thread loads, at a clamped token, so that the loads carry no
    // lane mask; only threads < ntok keep the result)
    auto fetch_positions = [&]() {
        const int t = t_first + max(min(tid, ntok - 1), 0);
        // without rotated dims positions are not read and never suppress
        const bool use_pos = a.rot > 0 && a.T > 0;
        const bool use_slot = !a.paged && !a.redirect && a.T > 0;
        const int64_t* pp = use_pos ? a.positions + t : reinterpret_cast<const int64_t*>(g_zero_row);
        const int64_t* sp = use_slot ? a.slot_mapping + t : reinterpret_cast<const int64_t*>(g_zero_row);
        const int64_t pv = gld(pp), sv = gld(sp);
        return TokMeta{use_pos ? pv : 0, use_slot ? sv : -1};
    };
    auto store_positions = [&](const TokMeta& m) {
        if (tid < ntok) {
            const int t = t_first + tid;
            s_pos[tid] = (a.rot == 0 || (m.pos >= 0 && m.pos < a.cs_rows)) ? (int)m.pos : -1;
            if (!a.paged) {
                int64_t koff = -1, voff = -1, srow = -1;
                if (a.redirect) {
                    koff = voff = (int64_t)t * a.kv_out_stride;
                    srow = t;
                } else if (m.slot >= 0 && m.slot < (int64_t)a.num_pages * a.page_size) {
                    // (slot < num_pages * page_size: 31 bits when the pool has fewer slots)
                    int64_t page, row;
                    if ((int64_t)a.num_pages * a.page_size <= INT32_MAX) {
                        page = fdiv31((int)m.slot, a.ps_div);
                        row = m.slot - page * a.page_size;
                    } else {
                        page = m.slot / a.page_size;
                        row = m.slot % a.page_size;
                    }
                    koff = page * a.k_page_stride + row * row_elems;
                    voff = page * a.v_page_stride + row * row_elems;
                    srow = m.slot;
                }
                s_koff[tid] = koff;
                s_voff[tid] = voff;
                s_srow[tid] = srow;
                s_qsoff[tid] = (int64_t)t * a.Hq;
            }
        }
    };
    auto stage_positions = [&]() { store_positions(fetch_positions()); };
    // request lookup, page and cos/sin row of every tile token (needs s_pos):
    // all loads issued first (unmasked, at clamped indices or from the zero
    // row), then the LDS writes, so that the tile costs one round trip
    constexpr int NCS = (kMaxTokensPerTile * D4 + kBlockThreads - 1) / kBlockThreads;   // float4 per thread
    struct RowsFetch {
        float4 cs[NCS];
        int64_t page;
        int b, j, L;
    };
    auto fetch_rows = [&]() {
        RowsFetch f;
#pragma unroll
        for (int n = 0; n < NCS; ++n) {
            // (the round count is the same for the whole workgroup)
            if (n > 0 && n * kBlockThreads >= ntok * D4) break;
            const int k = tid + n * kBlockThreads;
            const int i = min(k / D4, kMaxTokensPerTile - 1);
            const int c4 = k - (k / D4) * D4;
            const int p = s_pos[i];
            const bool ok = k < ntok * D4 && p >= 0 && 4 * c4 < a.rot;
            f.cs[n] = ldf4(ok ? a.cos_sin + (int64_t)p * a.rot + 4 * c4 : reinterpret_cast<const float*>(g_zero_row));
        }
        // Indices are clamped so that malformed metadata (rejected by the
        // verdict computed alongside) still reads inside the page table; only
        // the load address is selected, so that no branch surrounds the load.
        const int ti = max(min(tid, ntok - 1), 0);
        const int t = t_first + ti;
        f.b = f.j = f.L = 0;
        if (a.paged) {
            const int b = max(min(s_treq[ti], a.B - 1), 0);
            const int beg = s_indptr[b];
            const int ql = s_indptr[b + 1] - beg;
            f.b = b;
            f.j = t - beg;
            f.L = s_seqlen[b] - ql + f.j;
        }
        const int pidx = min(max(fdiv31(max(f.L, 0), a.ps_div), 0), a.maxp - 1);
        const bool use = a.paged && !a.redirect;
        f.page = gld(use ? a.page_table + (int64_t)f.b * a.maxp + pidx : reinterpret_cast<const int*>(g_zero_row));
        return f;
    };
    auto store_rows = [&](const RowsFetch& f) {
#pragma unroll
        for (int n = 0; n < NCS; ++n) {
            const int k = tid + n * kBlockThreads;
            const int i = k / D4;
            const int c4 = k - i * D4;
            if (k < ntok * D4 && s_pos[i] >= 0 && 4 * c4 < a.rot)
                *reinterpret_cast<float4*>(s_cs + i * D + 4 * c4) = f.cs[n];
        }
        if (a.paged && tid < ntok) {
            const int t = t_first + tid;
            if (a.redirect) {
                s_koff[tid] = s_voff[tid] = (int64_t)t * a.kv_out_stride;
                s_srow[tid] = t;
            } else {
                const int64_t row = f.L - fdiv31(max(f.L, 0), a.ps_div) * a.page_size;
                s_koff[tid] = f.page * a.k_page_stride + row * row_elems;
                s_voff[tid] = f.page * a.v_page_stride + row * row_elems;
                s_srow[tid] = f.page * a.page_size + row;
            }
            s_qsoff[tid] = a.q_scale_padded ? (int64_t)f.b * a.Hq * a.q_scale_P + f.j : (int64_t)t * a.Hq;
        }
    };
    auto stage_rows = [&]() { store_rows(fetch_rows()); };

    // Requests of this workgroup (flags, and tail clears when there are more
    // requests than workgroups).  With at least as many workgroups as
    // requests, the tail of request blockIdx % B is instead split across all
    // workgroups with that index: one workgroup clearing a whole 64-row
    // page tail would start its token items late and end the kernel late.
    // (B * (grid + 1) < 2^31: B <= kMaxRequests)
    const int r_lo = fdiv31(a.B * (int)blockIdx.x, a.grid_div);
    const int r_hi = fdiv31(a.B * ((int)blockIdx.x + 1), a.grid_div);
    const bool tail_spread = a.paged && a.B <= a.grid;
    const int bq = fdiv31((int)blockIdx.x, a.b_div);
    const int t_req = tail_spread ? (int)blockIdx.x - bq * a.B : 0;
    const int t_slice = tail_spread ? bq : 0;
    const int t_nslices = tail_spread ? fdiv31(a.grid - 1 - t_req, a.b_div) + 1 : 1;
    // page ids of the tails this workgroup clears (first kTailPrefetch requests)
    auto fetch_tail = [&]() {
        const int b = tail_spread ? t_req : min(r_lo + tid, max(r_hi - 1, 0));
        const int sl = a.paged ? s_seqlen[min(b, a.B - 1)] : 0;
        const int pidx = min(fdiv31(max(sl - 1, 0), a.ps_div), a.maxp - 1);
        const bool use = a.paged && a.zero_tail && sl > 0;
        return gld(use ? a.page_table + (int64_t)b * a.maxp + pidx : reinterpret_cast<const int*>(g_zero_row));
    };
    auto store_tail = [&](int page) {
        const int b = tail_spread ? t_req : r_lo + tid;
        if (tid < kTailPrefetch && (tail_spread ? tid == 0 : b < r_hi))
            s_tail[tid] = (a.zero_tail && s_seqlen[b] > 0) ? page : -1;
    };

    // Device scalars of the call: the loads are issued here, with the first
    // round of metadata, and the values are first used after its barrier
    // (a reciprocal taken right away would wait for them on the spot).
    const float k_scale_v = (KVFP8 && a.kv_group == 0) ? *a.k_scale : 1.0f;
    const float v_scale_v = (KVFP8 && a.kv_group == 0) ? *a.v_scale : 1.0f;
    const float q_static_v = (QMODE == 2) ? *a.q_scale_inv : 1.0f;
    RowConsts kc;
    kc.kv_ng = a.kv_group ? D / a.kv_group : 0;
    kc.inv_um = (QMODE == 1) ? 1.0f / a.upper_max : 1.0f;
    kc.qs_hstride = a.q_scale_padded ? (int)a.q_scale_P : 1;
    // Padded scales of consecutive tokens are 4-byte neighbours in each head's
    // row: written one by one they cost a partial-sector memory write each,
    // so they are gathered per tile in LDS and written as contiguous runs.
    kc.s_qs = (QMODE == 1 && a.stage_q_scale)
                  ? reinterpret_cast<float*>(s_dyn + ((3 * a.B + 2 + 3) & ~3)) : nullptr;

    // ---- first tile: its qkv loads go out with the first metadata round ----
    // The request metadata, the norm weights and the tile's positions are
    // loaded into registers first and the first qkv batch right after them:
    // load counters retire in order, so waiting for the metadata then does
    // not wait for the (much larger) qkv batch.
    const bool have_items = next_range();
    sub_lo = blo;
    if (have_items) start_tile();
    constexpr int WPT = (2 * D + kBlockThreads - 1) / kBlockThreads;   // norm weights per thread
    {
        // unmasked loads at clamped indices or from the zero row (a paged
        // launch has B >= 1); request metadata up to 512 requests here
        const float* zf = reinterpret_cast<const float*>(g_zero_row);
        const int* zi = reinterpret_cast<const int*>(g_zero_row);
        float wr[WPT];
#pragma unroll
        for (int k = 0; k < WPT; ++k) {
            const int i = min(tid + k * kBlockThreads, 2 * D - 1);
            wr[k] = gld(a.norm != 0 ? (i < D ? a.q_w + i : a.k_w + (i - D)) : zf);
        }
        int ip[2], sl[2];
#pragma unroll
        for (int k = 0; k < 2; ++k) {
            const int i = tid + k * kBlockThreads;
            ip[k] = gld(a.paged ? a.q_indptr + min(i, a.B) : zi);
            sl[k] = gld(a.paged ? a.seq_lens + min(i, a.B - 1) : zi);
        }
        const TokMeta m = fetch_positions();
        load_batch(bufA);   // rows of token 0 (or zeros) when this workgroup has no items
        const float add = (a.norm == 2) ? 1.0f : 0.0f;
#pragma unroll
        for (int k = 0; k < WPT; ++k) {
            const int i = tid + k * kBlockThreads;
            if (a.norm != 0 && i < 2 * D) s_w[i] = wr[k] + add;
        }
        if (a.paged) {
#pragma unroll
            for (int k = 0; k < 2; ++k) {
                const int i = tid + k * kBlockThreads;
                if (i <= a.B) s_indptr[i] = ip[k];
                if (i < a.B) s_seqlen[i] = sl[k];
            }
            for (int i = tid + 2 * kBlockThreads; i <= a.B; i += kBlockThreads) s_indptr[i] = a.q_indptr[i];
            for (int i = tid + 2 * kBlockThreads; i < a.B; i += kBlockThreads) s_seqlen[i] = a.seq_lens[i];
        }
        if (have_items) store_positions(m);
    }
    __syncthreads();
    kc.inv_k = 1.0f / k_scale_v;
    kc.inv_v = 1.0f / v_scale_v;
    kc.q_static = q_static_v;
    int bad = 0;
    Verdict vd{0, 0, 0, 0, 0};
    if (a.paged) {
        // (the first tile's token -> request map is written in the same
        // pass; the barriers inside make it visible)
        vd = validate_requests(a, s_indptr, s_seqlen, s_pre, s_wave, s_vote, s_pgreq, s_pgcol, s_vpre, s_treq,
                               t_first, have_items ? ntok : 0);
        bad = vd.bad;
    }
    {
        // The page-id checks, the tile's row lookups and cos/sin loads and the
        // tail-page prefetch are independent and all issue at once.  Page
        // reads stay inside the page table even for malformed metadata (the
        // page counts of an inconsistent request are zero and the row lookups
        // are clamped); nothing is written unless the whole call is valid.
        const int total_pages = (a.paged && !vd.fast) ? s_pre[a.B] : 0;
        // Calls that write more pages than threads read the ids in a second
        // round anyway; there the vector walk below checks every page.  Up to
        // kBlockThreads pages, one id per thread in this round is cheaper.
        const bool vec = a.pt_vec && total_pages > kBlockThreads;
        const int ks = min(tid, max(min(total_pages, kPageSlots) - 1, 0));
        const int* pp = reinterpret_cast<const int*>(g_zero_row);
        if (total_pages > 0 && !vec)
            pp = a.B > kSearchRequests ? a.page_table + (int64_t)s_pgreq[ks] * a.maxp + s_pgcol[ks]
                                       : page_id_ptr(a, s_indptr, s_seqlen, s_pre, ks);
        const int p_first = gld(pp);
        const RowsFetch rf = fetch_rows();
        const int tail_page = fetch_tail();
        // (the vector walk's first loads go out while the lookups above are in flight)
        if (vec) bad |= page_vectors_out_of_pool(a, s_indptr, s_seqlen, s_vpre);
        if (have_items) store_rows(rf);
        if (a.paged) store_tail(tail_page);
        if (vd.npg >= 1) bad |= page_out_of_pool(a, vd.pg0);
        if (vd.npg >= 2) bad |= page_out_of_pool(a, vd.pg1);
        if (!vec) {
            if (tid < total_pages) bad |= page_out_of_pool(a, p_first);
            if (total_pages > kBlockThreads)
                bad |= pages_out_of_pool(a, s_indptr, s_seqlen, s_pre, tid + kBlockThreads, total_pages);
        }
    }
    bad = block_or4(bad, s_flag);


    auto run_batch = [&](uint4 (&buf)[U][2]) {
#pragma unroll
        for (int u = 0; u < U; ++u) {
            if (pr.left > 0) {
                // (all lanes active here)
                if constexpr (kPairRows) mirror_exchange<kDppRowHalfMirror, 0xA, 0x5>(buf[u][0], buf[u][1]);
                if constexpr (PART && D == 128) {
                    if (half_rot) mirror_exchange<kDppRowHalfMirror, 0xA, 0x5>(buf[u][0], buf[u][1]);
                    else if (wide_rot) mirror_exchange_sel<kDppRowHalfMirror>(buf[u][0], buf[u][1], xhi, xlo);
                }
                if constexpr (PART && D == 256) {
                    if (half_rot) mirror_exchange<kDppRowMirror, 0xC, 0x3>(buf[u][0], buf[u][1]);
                    else if (wide_rot) mirror_exchange_sel<kDppRowMirror>(buf[u][0], buf[u][1], xhi, xlo);
                }
                const int r = pr.c * RPW + grp;
                const int ti = pr.t - t_first;
                if (r < a.R && s_pos[ti] >= 0)
                    process_row<D, QMODE, KVFP8, NTS>(a, pr.t, ti, r, gl, lm, buf[u][0], buf[u][1], s_w,
                                                 s_cs + ti * D, s_koff, s_voff, s_qsoff, s_srow, kc);
                pr.advance(CPT);
            }
        }
    };

    // ------------------ requests: flags and tail clear ------------------
    // (issued before the token items so the zero stores drain while the
    // rows are processed)
    // slice `slice` of `nslices` of the tail rows of request b (seq_len sl > 0):
    // the 4 KiB pieces slice, slice + nslices, ... (whole lines, no division)
    auto clear_tail = [&](int sl, int64_t page, int slice, int nslices) {
        const int pcol = fdiv31(sl - 1, a.ps_div);
        const int last = (sl - 1) - pcol * a.page_size;
        const int64_t nvec = (int64_t)(a.page_size - 1 - last) * row_elems * (int64_t)sizeof(kv_t) / 16;
        char* kb = reinterpret_cast<char*>(reinterpret_cast<kv_t*>(a.k_cache) + page * a.k_page_stride +
                                           (last + 1) * row_elems);
        char* vb = reinterpret_cast<char*>(reinterpret_cast<kv_t*>(a.v_cache) + page * a.v_page_stride +
                                           (last + 1) * row_elems);
        const uint4 z = make_uint4(0, 0, 0, 0);
        for (int64_t i = (int64_t)slice * kBlockThreads + tid; i < nvec; i += (int64_t)kBlockThreads * nslices) {
            st16_stream(kb + 16 * i, z);
            st16_stream(vb + 16 * i, z);
        }
        if (kc.kv_ng) {
            // the cleared rows' dynamic scales
            const int64_t ns = (int64_t)a.Hkv * kc.kv_ng;
            const int64_t first = (page * a.page_size + last + 1) * ns;
            const int64_t cnt = (int64_t)(a.page_size - 1 - last) * ns;
            for (int64_t i = (int64_t)slice * kBlockThreads + tid; i < cnt; i += (int64_t)kBlockThreads * nslices) {
                a.k_scale_out[first + i] = 0.0f;
                a.v_scale_out[first + i] = 0.0f;
            }
        }
    };
    // Flags of this workgroup's requests, then the tail clears: before the
    // token rows (their zero stores drain while the rows are processed) or,
    // in the TL instances, after them (one copy in each instance).
#define QKPREP_NRA_FLAGS_AND_TAILS()                                                                      \
    for (int b = r_lo; a.paged && b < r_hi; ++b) {                                                        \
        for (int h = tid; h < a.Hkv; h += kBlockThreads) a.flags[(int64_t)b * a.Hkv + h] = bad ? -1 : 0;  \
        if (bad || !a.zero_tail || tail_spread) continue;                                                 \
        const int sl = s_seqlen[b];                                                                       \
        if (sl <= 0) continue;                                                                            \
        /* (an LDS read for the prefetched pages; a select between the two                                \
        would become a flat load whose wait drains every store in flight) */                              \
        int64_t page;                                                                                     \
        if (b - r_lo < kTailPrefetch)                                                                     \
            page = s_tail[b - r_lo];                                                                      \
        else                                                                                              \
            page = gld(a.page_table + (int64_t)b * a.maxp + fdiv31(sl - 1, a.ps_div));                    \
        clear_tail(sl, page, 0, 1);                                                                       \
    }                                                                                                     \
    if (tail_spread && !bad && a.zero_tail && s_seqlen[t_req] > 0)                                        \
        clear_tail(s_seqlen[t_req], s_tail[0], t_slice, t_nslices);
    if constexpr (!TL) {
        QKPREP_NRA_FLAGS_AND_TAILS();
    }

    // ---------------------------- token items ----------------------------
    if (have_items && !bad) {
        for (;;) {
            // double-buffered: the next batch's loads are issued before the
            // current batch's stores
            while (pr.left > 0) {
                load_batch(bufB);
                run_batch(bufA);
                if (pr.left <= 0) break;
                load_batch(bufA);
                run_batch(bufB);
            }
            if (kc.s_qs) {
                // each head's scales of the tile's tokens, token-contiguous;
                // only the heads whose chunks lie in this workgroup's range
                // (the first and last token may be shared with a neighbour)
                __syncthreads();
                const int c_first = sub_lo - t_first * CPT;            // first chunk of token 0
                const int c_last = sub_hi - (t_first + ntok - 1) * CPT; // end chunk of the last token
                for (int k = tid; k < ntok * a.Hq; k += kBlockThreads) {
                    const int h = k / ntok;
                    const int i = k - h * ntok;
                    const int c = h / RPW;
                    const bool mine = (i > 0 || c >= c_first) && (i < ntok - 1 || c < c_last);
                    if (mine && s_pos[i] >= 0)
                        a.q_scale[s_qsoff[i] + (int64_t)h * a.q_scale_P] = kc.s_qs[i * a.Hq + h];
                }
            }
            sub_lo = sub_hi;
            if (sub_lo >= bhi) {
                if (!next_range()) break;
                sub_lo = blo;
            }
            start_tile();
            // positions first, then the qkv batch: the wait for the positions
            // (load counters retire in order) then excludes the batch
            const TokMeta m = fetch_positions();
            load_batch(bufA);
            __syncthreads();   // every wave is done with the previous tile's LDS rows
            store_positions(m);
            if (a.paged) scatter_tokens();
            __syncthreads();
            stage_rows();
            __syncthreads();
        }
    }
    if constexpr (TL) {
        QKPREP_NRA_FLAGS_AND_TAILS();
    }
#undef QKPREP_NRA_FLAGS_AND_TAILS
}

template <int D, int QMODE, bool KVFP8, int ROT, int MEM>
hipError_t launch_t(const NraDevArgs& a, hipStream_t stream) {
    size_t lds = a.paged ? (size_t)(3 * a.B + 2) * sizeof(int) : 0;
    if (a.stage_q_scale) lds = (size_t)((3 * a.B + 2 + 3) & ~3) * sizeof(int) + (size_t)kMaxTokensPerTile * a.Hq * sizeof(float);
    // enough workgroups to fill every CU, none with less than 8 head-row
    // chunks of work, and at least one per request when tails are cleared
    // (one per 4 requests otherwise, for the flags)
    int64_t cap = resident_grid(reinterpret_cast<const void*>(&nra_kernel<D, QMODE, KVFP8, ROT, MEM, false>), lds);
    if (cap < 1) cap = 256;
    // 8 (token, chunk) items per workgroup, but 4 for small calls (up to 64
    // workgroups): a tiny decode's time is its latency chain, which more
    // workgroups shorten (16 tokens: 9.4 -> 8.1 us), while at B = 256 the
    // 8-item split measured best.  A decode with few head rows per token and
    // long tails (8/1 heads, page 64, 256 requests) otherwise gives each
    // workgroup four requests' tails: one per request took it from 14.8 to
    // 12.6 us.  With fewer requests than CUs, each request's tail is split
    // over B * floor(256 / B) workgroups (about one per CU of the 256), so
    // that the zero stores of a few long page tails leave from every CU
    // instead of a handful: the 1-request decode with a 63-row page-64 tail
    // 7.0 -> 6.6 us, 32 requests with 64/8 heads 8.2 -> 7.3, the 16-token
    // decode 6.3 -> 6.0; neutral from 128 requests up.
    int64_t want = (a.total_items + 7) / 8;
    const int64_t want4 = (a.total_items + 3) / 4;
    if (want < (want4 < 64 ? want4 : 64)) want = want4 < 64 ? want4 : 64;
    const int64_t per_req = !a.zero_tail ? (a.B + 3) / 4
                            : (a.B > 0 && a.B < kTailSpreadGroups) ? (int64_t)a.B * (kTailSpreadGroups / a.B)
                                                                   : a.B;
    if (want < per_req) want = per_req;
    if (want < 1) want = 1;
    NraDevArgs la = a;
    la.grid = (int)(want < cap ? want : cap);
    // Long calls (8 or more tokens per workgroup) deal spans of 24 (token,
    // chunk) items round-robin, not aligned to tokens: the resident
    // workgroups then stream through one narrow window of qkv and the caches
    // instead of the whole call at once.  With rotating buffers (the previous
    // calls' outputs still being written back) 24-item spans measured best
    // or near best on every prefill shape: the 15k-token FP8 prefill 96.4 ->
    // 88.5 us against 4-token spans (40 items), the 16k one 103.6 -> 95.8,
    // 64-dim heads 52.5 -> 51.4, the strided 256-dim one 50.8 -> 49.3; 20 to
    // 32 items are close, 12 or 16 items slower (the per-tile metadata round
    // then dominates), 48 slower.  Spans are dealt to the XCDs in runs of
    // kXcdRun (see next_range): runs of 16 or 32 spans took the 16k-token
    // prefill from 90.9 to 87.4 us and the T = 14 876 draw from 83.5 to
    // 81.2 us, while runs of 64 or 128 (each XCD a contiguous eighth of the
    // round) were slower than none.  Short calls keep one contiguous range
    // each.
    la.interleave = (a.T >= 8 * (int64_t)la.grid) ? 24 : 0;
    la.grid_div = make_fastdiv31((uint32_t)la.grid);
    la.cpt_div = make_fastdiv31((uint32_t)(a.chunks_per_token > 0 ? a.chunks_per_token : 1));
    la.b_div = make_fastdiv31((uint32_t)(a.B > 0 ? a.B : 1));
    la.items_q = (int)(a.total_items / la.grid);
    la.items_r = (int)(a.total_items % la.grid);
    (void)hipGetLastError();   // the status below then covers this launch only
    // Decodes of many requests with several head-row chunks per token clear
    // the tails after the token rows (TL instances, whole-head rotary and
    // streaming Q stores only): there the tails' stores otherwise delay the
    // rows.  B = 256 decodes: 32/8 heads page 16 7.9 -> 7.6 us, 64/8 heads
    // page 64 15.0 -> 13.4 us; smaller calls lose from it (their time is the
    // latency chain plus one tail drain), 8/1 heads (two chunks) gain nothing.
    if constexpr (ROT == kRotWhole && MEM == kMemStream) {
        if (la.interleave == 0 && a.zero_tail && a.B >= kTailsLastRequests && a.chunks_per_token >= 4) {
            hipLaunchKernelGGL((nra_kernel<D, QMODE, KVFP8, ROT, MEM, true>), dim3(la.grid), dim3(kBlockThreads), lds,
                               stream, la);
            return hipGetLastError();
        }
    }
    hipLaunchKernelGGL((nra_kernel<D, QMODE, KVFP8, ROT, MEM, false>), dim3(la.grid), dim3(kBlockThreads), lds, stream, la);
    return hipGetLastError();
}

}  // namespace

#ifndef QKPREP_NRA_HEAD_DIM
#error "nra_kernel.hip is compiled once per head dim with -DQKPREP_NRA_HEAD_DIM=64, 128 or 256"
#endif
#define QKPREP_CAT2(x, y) x##y
#define QKPREP_CAT(x, y) QKPREP_CAT2(x, y)

// Launch for head dim QKPREP_NRA_HEAD_DIM: picks the instance for the Q mode,
// the cache dtype, the rotary layout (whole head, partial, none) and the
// memory mode (in place: cached loads and stores; streaming loads with
// streaming or ordinary row stores).  A call without rotated dims takes the
// whole-head lane layout, whose load instructions read whole lines.
hipError_t QKPREP_CAT(launch_norm_rope_append_d, QKPREP_NRA_HEAD_DIM)(const NraDevArgs& a, int q_mode, int kv_fp8,
                                                                       hipStream_t stream) {
    constexpr int D = QKPREP_NRA_HEAD_DIM;
#define QKPREP_NRA_ROT(QM, KF, RT)                                                                       \
    switch (a.mem) {                                                                                     \
        case kMemInPlace: return launch_t<D, QM, KF, RT, kMemInPlace>(a, stream);                          \
        case kMemStream: return launch_t<D, QM, KF, RT, kMemStream>(a, stream);                            \
        default: return launch_t<D, QM, KF, RT, kMemKeep>(a, stream);                                      \
    }
#define QKPREP_NRA_CASE(QM, KF)                                                                          \
    if (q_mode == QM && (kv_fp8 != 0) == KF) {                                                           \
        if (a.rot == D) QKPREP_NRA_ROT(QM, KF, kRotWhole)                                                \
        if (a.rot == 0) QKPREP_NRA_ROT(QM, KF, kRotNone)                                                 \
        QKPREP_NRA_ROT(QM, KF, kRotPart)                                                                 \
    }
    QKPREP_NRA_CASE(0, false) QKPREP_NRA_CASE(0, true)
    QKPREP_NRA_CASE(1, false) QKPREP_NRA_CASE(1, true)
    QKPREP_NRA_CASE(2, false) QKPREP_NRA_CASE(2, true)
#undef QKPREP_NRA_ROT
#undef QKPREP_NRA_CASE
    return hipErrorInvalidValue;
}

}  // namespace qkprep
