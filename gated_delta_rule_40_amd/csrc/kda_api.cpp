// kda_api.cpp -- host side of the libkda C ABI (declared in include/kda.h).
//
// Validates every argument before touching HIP, picks the kernel tiling and
// launches on the caller's stream.  No device memory is allocated, no stream
// is synchronised and no mutable state is shared between calls.
#include <hip/hip_runtime.h>

#include <atomic>
#include <cstdint>
#include <cstdlib>
#include <cstring>
#include <mutex>
#include <vector>

#include "kda.h"

extern "C" hipError_t kda_launch_prefill(int bf16, int chunk, int dv_block, const void *q,
                                         const void *k, const void *v, const float *g,
                                         const float *beta, const float *init, const int32_t *cu,
                                         int32_t N, int32_t T_tot, int32_t H, int32_t dv,
                                         void *out, float *fin, float *snap, int32_t snap_every,
                                         int32_t max_snaps, const int32_t *snap_chunk_off, hipStream_t stream);
extern "C" hipError_t kda_launch_cp_plan_prep(int bf16, const void *q, const void *k, const float *g,
                                              const float *beta, const int32_t *cu, int32_t N, int32_t T_tot,
                                              int32_t H, int64_t max_chunks, void *img, void *gimg,
                                              int32_t seg_len, int32_t max_segs, int32_t *plan, int32_t *seq_seg,
                                              int32_t *chunk_off, int32_t *sched, int32_t last_len,
                                              int32_t skip_last, int32_t *seq_order, int32_t seg_len2,
                                              int32_t max_segs2, int32_t *plan2, int32_t *seq_seg2,
                                              int32_t *sched2, int32_t last_len2, int32_t skip_last2,
                                              int32_t *seq_order2, int32_t pieces, int32_t piece_len,
                                              hipStream_t stream);
extern "C" hipError_t kda_launch_chain(int bf16, int dv_block, const void *v, const float *init, const int32_t *cu, int32_t N,
                                       int32_t T_tot, int32_t H, int32_t dv, void *out, float *fin,
                                       const int32_t *plan, int32_t num_segs, int32_t mode, const float *seg_init,
                                       float *seg_out, const int32_t *chunk_off, const void *img,
                                       const int32_t *sched, void *snap, float *snap_scale, float *uw_u,
                                       float *uw_w, const int32_t *init_seq_seg, int32_t init_unit,
                                       int32_t init_units, int32_t cmb_fmt, int32_t narrow, int32_t init_tiles,
                                       int32_t sum_tail, int32_t pieces, int32_t *head_dead, int32_t sum_head,
                                       hipStream_t stream);
extern "C" size_t kda_chunk_image_bytes(int bf16);
extern "C" hipError_t kda_launch_grad_chain(int bf16, int summary, const void *dout, const int32_t *cu, int32_t N,
                                            int32_t T_tot, int32_t H, const int32_t *plan, int32_t num_segs,
                                            const int32_t *sched, const int32_t *chunk_off, const void *gimg,
                                            const float *g_end, void *g_chunk, float *g_scale, float *dinit,
                                            float *g0_out, float *dx_chunk, int32_t tiles,
                                            const int32_t *head_dead, int32_t sum_head, hipStream_t stream);
extern "C" hipError_t kda_launch_bwd_chunk(int bf16, const void *q, const void *k, const float *g,
                                           const float *beta, const void *dout, const int32_t *cu,
                                           const int32_t *chunk_off, int64_t max_chunks, const void *snaps,
                                           const float *snap_scale, const void *gchunk, const float *g_scale,
                                           const float *uw_u, const float *uw_w, const float *dx_chunk, int32_t N,
                                           int32_t T_tot, int32_t H, float *dq, float *dk, float *dv, float *dg,
                                           float *dbeta, hipStream_t stream);
extern "C" hipError_t kda_launch_decode_tokens(int bf16, const void *q, const void *k, const void *v,
                                               const float *g, const float *beta, const int32_t *cu,
                                               const int32_t *num_tokens, const float *state_in,
                                               float *state_out, int32_t N, int32_t T_tot, int32_t H, void *out,
                                               hipStream_t stream);
extern "C" hipError_t kda_launch_cp_combine(const float *init, int32_t N, int32_t H, int32_t dv,
                                            const int32_t *seq_seg, const float *seg_out, float *seg_init,
                                            int32_t reverse, const int32_t *plan, const int32_t *seq_order,
                                            const float *m_src, int32_t m_trans, int32_t fmt, hipStream_t stream);
extern "C" hipError_t kda_launch_decode(int bf16, const void *q, const void *k, const void *v,
                                        const float *g, const float *beta, float *state,
                                        int32_t N, int32_t H, void *out, hipStream_t stream);
extern "C" hipError_t kda_static_scratch(void **ptr, size_t *bytes);

namespace {

constexpr int32_t kHeadDim = 128;

bool aligned(const void *p, uintptr_t a) { return (reinterpret_cast<uintptr_t>(p) % a) == 0; }

kda_status check_common(const void *q, const void *k, const void *v, const float *g,
                        const float *beta, const void *out, int32_t dk, int32_t dv,
                        kda_dtype dtype)
{
    if (!q || !k || !v || !g || !beta || !out) return KDA_ERR_INVALID_ARG;
    if (dtype != KDA_F32 && dtype != KDA_BF16) return KDA_ERR_INVALID_ARG;
    if (dk <= 0 || dv <= 0) return KDA_ERR_INVALID_ARG;
    // 16-byte vector accesses on q, k, v, out and g rows
    if (!aligned(q, 16) || !aligned(k, 16) || !aligned(v, 16) || !aligned(out, 16) || !aligned(g, 16) ||
        !aligned(beta, 4))
        return KDA_ERR_INVALID_ARG;
    if (dk != kHeadDim || dv != kHeadDim) return KDA_ERR_UNSUPPORTED;
    return KDA_OK;
}

// KDA_VALIDATE=1 in the environment (read once): the entry points that take
// cu_seqlens copy it to the host, synchronising `stream`, and check it before
// launching anything.  Off by default, since it costs a synchronisation.
bool validate_enabled()
{
    static std::atomic<int> state{-1};
    int v = state.load(std::memory_order_relaxed);
    if (v < 0) {
        const char *e = std::getenv("KDA_VALIDATE");
        v = (e && std::strcmp(e, "1") == 0) ? 1 : 0;
        state.store(v, std::memory_order_relaxed);
    }
    return v == 1;
}

// cu[0] = 0, non-decreasing, cu[N] <= T.  Returns KDA_ERR_INVALID_ARG for
// contents that break this, KDA_ERR_LAUNCH if the copy itself fails.
kda_status validate_cu(const int32_t *cu, int32_t N, int32_t T, hipStream_t stream)
{
    std::vector<int32_t> h((size_t)N + 1);
    if (hipMemcpyAsync(h.data(), cu, sizeof(int32_t) * h.size(), hipMemcpyDeviceToHost, stream) != hipSuccess ||
        hipStreamSynchronize(stream) != hipSuccess)
        return KDA_ERR_LAUNCH;
    if (h[0] != 0 || h[N] > T) return KDA_ERR_INVALID_ARG;
    for (int32_t n = 0; n < N; ++n)
        if (h[n + 1] < h[n]) return KDA_ERR_INVALID_ARG;
    return KDA_OK;
}

// Value-column block per workgroup: the largest block that still gives at
// least one workgroup per compute unit, but not below 64 columns (more
// blocks = more parallel state chains, at the cost of repeating the
// state-independent chunk work; below 64 columns, i.e. four waves, that work
// is shared by too few waves and each chunk takes longer: 4,096 tokens x 8
// heads take 0.72 ms at 64 or 128 columns, 0.95 ms at 32 and 1.39 ms at 16).
int auto_dv_block(int64_t units, int dv)
{
    int cus = 256;
    int dev = 0;
    if (hipGetDevice(&dev) == hipSuccess) {
        int n = 0;
        if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) == hipSuccess && n > 0) cus = n;
    }
    int bv = dv;
    while (bv > 64 && units * (dv / bv) < cus) bv /= 2;
    return bv;
}

}  // namespace

extern "C" {

static kda_status prefill_impl(const void *q, const void *k, const void *v, const float *g,
                               const float *beta, const float *initial_state, const int32_t *cu_seqlens,
                               int32_t num_seqs, int32_t total_tokens, int32_t num_heads, int32_t dk,
                               int32_t dv, kda_dtype dtype, void *out, float *final_state,
                               int32_t chunk, int32_t dv_block, float *snap, int32_t snap_every,
                               int32_t max_snaps, kda_stream_t stream)
{
    kda_status st = check_common(q, k, v, g, beta, out, dk, dv, dtype);
    if (st == KDA_ERR_INVALID_ARG) return st;
    if (!cu_seqlens || num_seqs < 0 || total_tokens < 0 || num_heads <= 0) return KDA_ERR_INVALID_ARG;
    if (st != KDA_OK) return st;
    const bool bf16 = dtype == KDA_BF16;
    if (chunk == 0) chunk = 32;
    const bool chunk_ok = bf16 ? (chunk == 32 || chunk == 64) : (chunk == 16 || chunk == 32);
    if (!chunk_ok) return KDA_ERR_UNSUPPORTED;
    if (dv_block != 0 && dv_block != 16 && dv_block != 32 && dv_block != 64 && dv_block != 128)
        return KDA_ERR_UNSUPPORTED;
    if (dv_block > dv) return KDA_ERR_UNSUPPORTED;
    // 64-token bf16 chunks need at least two waves (value block >= 32)
    const int min_block = (bf16 && chunk == 64) ? 32 : 16;
    if (dv_block != 0 && dv_block < min_block) return KDA_ERR_UNSUPPORTED;
    if (snap) {
        if (snap_every <= 0 || max_snaps <= 0 || !aligned(snap, 4)) return KDA_ERR_INVALID_ARG;
        if (snap_every % chunk) return KDA_ERR_UNSUPPORTED;
    }
    const int64_t units = (int64_t)num_seqs * num_heads;
    if (units == 0) return KDA_OK;
    if (units * (dv / 16) > INT32_MAX) return KDA_ERR_INVALID_ARG;   // grid size
    if (validate_enabled())
        if (kda_status v = validate_cu(cu_seqlens, num_seqs, total_tokens, reinterpret_cast<hipStream_t>(stream)))
            return v;
    if (dv_block == 0) {
        dv_block = auto_dv_block(units, dv);
        if (dv_block < min_block) dv_block = min_block;
    }
    hipError_t e = kda_launch_prefill(bf16 ? 1 : 0, chunk, dv_block, q, k, v, g, beta, initial_state,
                                      cu_seqlens, num_seqs, total_tokens, num_heads, dv, out,
                                      final_state, snap, snap_every, max_snaps, nullptr,
                                      reinterpret_cast<hipStream_t>(stream));
    return e == hipSuccess ? KDA_OK : KDA_ERR_LAUNCH;
}

kda_status kda_prefill_ex(const void *q, const void *k, const void *v, const float *g,
                          const float *beta, const float *initial_state, const int32_t *cu_seqlens,
                          int32_t num_seqs, int32_t total_tokens, int32_t num_heads, int32_t dk,
                          int32_t dv, kda_dtype dtype, void *out, float *final_state,
                          int32_t chunk, int32_t dv_block, kda_stream_t stream)
{
    return prefill_impl(q, k, v, g, beta, initial_state, cu_seqlens, num_seqs, total_tokens, num_heads, dk, dv,
                        dtype, out, final_state, chunk, dv_block, nullptr, 0, 0, stream);
}

kda_status kda_prefill_snapshots(const void *q, const void *k, const void *v, const float *g,
                                 const float *beta, const float *initial_state, const int32_t *cu_seqlens,
                                 int32_t num_seqs, int32_t total_tokens, int32_t num_heads, int32_t dk,
                                 int32_t dv, kda_dtype dtype, void *out, float *final_state,
                                 int32_t snap_every, int32_t max_snaps, float *snapshots, kda_stream_t stream)
{
    if (!snapshots) return KDA_ERR_INVALID_ARG;
    return prefill_impl(q, k, v, g, beta, initial_state, cu_seqlens, num_seqs, total_tokens, num_heads, dk, dv,
                        dtype, out, final_state, 32, 64, snapshots, snap_every, max_snaps, stream);
}

kda_status kda_prefill(const void *q, const void *k, const void *v, const float *g,
                       const float *beta, const float *initial_state, const int32_t *cu_seqlens,
                       int32_t num_seqs, int32_t total_tokens, int32_t num_heads, int32_t dk,
                       int32_t dv, kda_dtype dtype, void *out, float *final_state,
                       kda_stream_t stream)
{
    return kda_prefill_ex(q, k, v, g, beta, initial_state, cu_seqlens, num_seqs, total_tokens,
                          num_heads, dk, dv, dtype, out, final_state, 0, 0, stream);
}

// ---------------------------------------------------------------- context parallel
namespace {

constexpr int32_t kCpChunk = 32;     // chunk size of the segmented runs
constexpr int32_t kCpBlock = 128;    // value columns per workgroup of the segment-output pass
constexpr int32_t kCpSumBlock = 256; // value + transition columns per workgroup of the summary pass
// chunks a summary unit is first walked over from its end: on decaying gates
// the transition over them is exactly zero in fp32, and the rest of the unit
// then cannot reach its end state (see the summary loop in kda_prefill.hip).
// Under g ~ U(-5/16, 0] the transition of a 256-chunk unit dies between 24
// and 36 chunks from its end: 16 and 24 sent most units back to a full walk
// (1M tokens x 16 heads: 17.7 ms), 32 some (13.7 ms), 36 almost none (13.3
// ms); longer tails only add work (44: 13.5 ms).
constexpr int32_t kCpSumTail = 36;
constexpr int64_t kNumCUs = 256;     // compute units of one MI355X

struct CpLayout {
    size_t plan, sched, seq_seg, uplan, usched, useq_seg, seq_order, chunk_off, seg_out, seg_init, img, total;
    int32_t max_segs, max_units, unit_len, max_chunks;
    // > 0: segments cut at the ends of pieces of the packed chunk order (at
    // most `pieces` per head, piece_len chunks each, or 0: equal pieces), one
    // output workgroup per (piece, head); units are then the segments
    int32_t pieces, piece_len;
};

size_t align256(size_t x) { return (x + 255) & ~size_t(255); }

// Summary units: when there are at least as many (segment, head) pairs as
// compute units (T / seg_len * H >= 256) and segments are long (at least
// 1,024 tokens), output segments (seg_len tokens) are
// cut into up to four units for the summary pass and the combine, so that the
// summary pass, one workgroup per (unit, head) at one per compute unit, is
// made of many short pieces that pack the GPU evenly; the output pass still
// runs whole segments, from the entering state of their first unit.  Below
// that the summary pass is a single round anyway, and more units would only
// lengthen the combine's chain.  The unit length divides seg_len and is a
// multiple of the chunk.  bf16 inputs keep whole segments: their summaries
// walk a unit's last kCpSumTail chunks when the transition over them is zero,
// so a summary no longer costs in proportion to its unit's length, and fewer
// units mean fewer summaries and a shorter combine chain (1M tokens x 16
// heads: 12.57 ms against 13.26 ms with quarter-segment units; 4 x 16,384 x
// 32: 1.64 against 1.82 ms).  When the transition does not die, the walks
// cover about the same chunks either way (a unit's tail plus the unit).
int32_t cp_unit_len(int32_t seg_len, int32_t T, int32_t H, int bf16)
{
    const int32_t m = seg_len / kCpChunk;
    if (bf16 || (int64_t)T / seg_len * H < 256 || seg_len < 1024) return seg_len;
    return m % 4 == 0 ? seg_len / 4 : (m % 2 == 0 ? seg_len / 2 : seg_len);
}

// Workspace sections: the output plan [max_segs][4] int32, its dispatch
// order [max_segs] int32 and per-sequence first segment [N + 1] int32; the
// same three for the summary units (max_units); the sequences by unit count
// [N] int32; per-sequence first chunk
// [N + 1] int32; summaries [max_units][H][dk][dv + dk] fp32; entering states
// [max_units][H][dk][dv] fp32; chunk-operand images [max_chunks][H][image].
// Every sequence of length L takes max(1, ceil(L / len)) segments (units) and
// ceil(L / 32) chunks, which max_segs, max_units and max_chunks bound.
// With pieces, a sequence takes one segment per piece its chunks reach (one
// when empty), so there are at most pieces + N segments.
bool cp_layout(int32_t N, int32_t T, int32_t H, int32_t dk, int32_t dv, int bf16, int32_t seg_len, int32_t pieces,
               int32_t piece_len, CpLayout *lay)
{
    const int32_t unit = pieces > 0 ? seg_len : cp_unit_len(seg_len, T, H, bf16);
    const int64_t segs = pieces > 0 ? (int64_t)pieces + 1 + N : (int64_t)T / seg_len + 1 + N;
    const int64_t units = pieces > 0 ? segs : (int64_t)T / unit + 1 + N;
    const int64_t chunks = (int64_t)T / kCpChunk + 1 + N;
    if (units > INT32_MAX / 4 || chunks > INT32_MAX / 4) return false;
    lay->pieces = pieces;
    lay->piece_len = piece_len;
    lay->max_segs = (int32_t)segs;
    lay->max_units = (int32_t)units;
    lay->unit_len = unit;
    lay->max_chunks = (int32_t)chunks;
    lay->plan = 0;
    lay->sched = align256(lay->plan + sizeof(int32_t) * 4 * (size_t)segs);
    lay->seq_seg = align256(lay->sched + sizeof(int32_t) * (size_t)segs);
    lay->uplan = align256(lay->seq_seg + sizeof(int32_t) * ((size_t)N + 1));
    lay->usched = align256(lay->uplan + sizeof(int32_t) * 4 * (size_t)units);
    lay->useq_seg = align256(lay->usched + sizeof(int32_t) * (size_t)units);
    lay->seq_order = align256(lay->useq_seg + sizeof(int32_t) * ((size_t)N + 1));
    lay->chunk_off = align256(lay->seq_order + sizeof(int32_t) * ((size_t)N + 1));
    lay->seg_out = align256(lay->chunk_off + sizeof(int32_t) * ((size_t)N + 1));
    lay->seg_init = align256(lay->seg_out + sizeof(float) * (size_t)units * H * dk * (dv + dk));
    lay->img = align256(lay->seg_init + sizeof(float) * (size_t)units * H * dk * dv);
    lay->total = align256(lay->img + kda_chunk_image_bytes(bf16) * (size_t)chunks * H);
    return true;
}

// Default segment length: about 256 (segment, head) pairs (one output-pass
// workgroup per compute unit: fewer, longer segments than two per unit, so
// fewer summary units and a shorter combine chain), at least 256 tokens (8
// chunks: shorter segments add more combine steps than they take off a
// workgroup's walk) and at most 32,768 (1,024 chunks: a longer segment's walk
// becomes the critical path).  Measured: 4,096 tokens x 8 heads take 0.133 ms
// at 256, 0.146 ms at 512 and 0.40 ms at 128; 4 x 16,384 tokens x 32 heads
// 1.9-2.0 ms at 8,192 against 2.13 ms at 4,096 and 16,384; the 1M-token
// varlen batch x 16 heads 17.0 ms at 32,768 against 17.3 ms at 16,384 and
// 18.0-18.1 ms at 49,152 and 65,536.
int32_t cp_default_seg_len(int32_t T, int32_t H)
{
    int64_t len = (int64_t)T * H / 256;
    len = len < 256 ? 256 : (len > 32768 ? 32768 : len);
    return (int32_t)((len + kCpChunk - 1) / kCpChunk * kCpChunk);
}

// The segment cut of a call: seg_len > 0 cuts every sequence into seg_len
// tokens from its start; seg_len < 0 cuts the packed chunk order into pieces
// of -seg_len tokens; 0 chooses.  Pieces are the
// automatic choice for 16-bit inputs and at most 256 sequences when the
// segments would be capped (T H / 256 above 32,768 tokens): then the fewest
// equal pieces that give every one of two workgroups per compute unit one
// piece (512 / H per head), so that every output walk has the same length.
// Cut per sequence, the 1M-token varlen batch (eight sequences, 16 heads)
// has 592 output workgroups of up to 1,024 chunks for 512 places, and the
// last ones start as the first finish.
kda_status cp_cut(int32_t N, int32_t T, int32_t H, int bf16, int32_t *seg_len, int32_t *pieces, int32_t *piece_len)
{
    *pieces = 0;
    *piece_len = 0;
    if (*seg_len < 0) {
        if (*seg_len < -(INT32_MAX / 2) || (-*seg_len) % kCpChunk) return KDA_ERR_UNSUPPORTED;
        *seg_len = -*seg_len;
        *piece_len = *seg_len / kCpChunk;
        const int64_t np = ((int64_t)T / kCpChunk + N + *piece_len - 1) / *piece_len;
        if (np > INT32_MAX / 8) return KDA_ERR_UNSUPPORTED;
        *pieces = (int32_t)(np > 0 ? np : 1);
        return KDA_OK;
    }
    if (*seg_len > 0) return *seg_len % kCpChunk ? KDA_ERR_UNSUPPORTED : KDA_OK;
    *seg_len = cp_default_seg_len(T, H);
    if (bf16 && N >= 1 && N <= 256 && (int64_t)T * H / 256 > 32768) {
        *pieces = (int32_t)(2 * kNumCUs / H > 1 ? 2 * kNumCUs / H : 1);
        *piece_len = 0;
    }
    return KDA_OK;
}

}  // namespace

size_t kda_prefill_cp_workspace_size(int32_t num_seqs, int32_t total_tokens, int32_t num_heads,
                                     int32_t dk, int32_t dv, kda_dtype dtype, int32_t seg_len)
{
    if (num_seqs < 0 || total_tokens < 0 || num_heads <= 0 || dk != kHeadDim || dv != kHeadDim) return 0;
    if (dtype != KDA_F32 && dtype != KDA_BF16) return 0;
    int32_t pieces, piece_len;
    if (cp_cut(num_seqs, total_tokens, num_heads, dtype == KDA_BF16, &seg_len, &pieces, &piece_len) != KDA_OK) return 0;
    if (seg_len < kCpChunk || seg_len % kCpChunk) return 0;
    CpLayout lay;
    if (!cp_layout(num_seqs, total_tokens, num_heads, dk, dv, dtype == KDA_BF16, seg_len, pieces, piece_len, &lay))
        return 0;
    return lay.total;
}

namespace {

// Argument checks of kda_prefill_cp and kda_prefill_cp_noalloc (no HIP call):
// resolves the automatic segment length and the workspace layout.
kda_status cp_check(const void *q, const void *k, const void *v, const float *g, const float *beta,
                    const int32_t *cu_seqlens, int32_t num_seqs, int32_t total_tokens, int32_t num_heads,
                    int32_t dk, int32_t dv, kda_dtype dtype, void *out, int32_t *seg_len, CpLayout *lay)
{
    kda_status st = check_common(q, k, v, g, beta, out, dk, dv, dtype);
    if (st == KDA_ERR_INVALID_ARG) return st;
    if (!cu_seqlens || num_seqs < 0 || total_tokens < 0 || num_heads <= 0) return KDA_ERR_INVALID_ARG;
    if (st != KDA_OK) return st;
    int32_t pieces, piece_len;
    if (kda_status c = cp_cut(num_seqs, total_tokens, num_heads, dtype == KDA_BF16, seg_len, &pieces, &piece_len))
        return c;
    if (*seg_len < kCpChunk || *seg_len % kCpChunk) return KDA_ERR_UNSUPPORTED;
    if (!cp_layout(num_seqs, total_tokens, num_heads, dk, dv, dtype == KDA_BF16, *seg_len, pieces, piece_len, lay))
        return KDA_ERR_INVALID_ARG;
    if ((int64_t)lay->max_units * num_heads * ((dv + dk) / 16) > INT32_MAX) return KDA_ERR_INVALID_ARG;
    if ((int64_t)lay->max_chunks * num_heads > INT32_MAX) return KDA_ERR_INVALID_ARG;
    return KDA_OK;
}

// The five launches of a context-parallel prefill in workspace `ws` (layout `lay`).
kda_status cp_launch(const void *q, const void *k, const void *v, const float *g, const float *beta,
                     const float *initial_state, const int32_t *cu_seqlens, int32_t num_seqs,
                     int32_t total_tokens, int32_t num_heads, int32_t dv, kda_dtype dtype, void *out,
                     float *final_state, int32_t seg_len, const CpLayout &lay, void *workspace, hipStream_t s)
{
    if (num_seqs == 0) return KDA_OK;
    const int bf16 = dtype == KDA_BF16 ? 1 : 0;
    char *ws = static_cast<char *>(workspace);
    int32_t *plan = reinterpret_cast<int32_t *>(ws + lay.plan);
    int32_t *sched = reinterpret_cast<int32_t *>(ws + lay.sched);
    int32_t *seq_seg = reinterpret_cast<int32_t *>(ws + lay.seq_seg);
    int32_t *uplan = reinterpret_cast<int32_t *>(ws + lay.uplan);
    int32_t *usched = reinterpret_cast<int32_t *>(ws + lay.usched);
    int32_t *useq_seg = reinterpret_cast<int32_t *>(ws + lay.useq_seg);
    int32_t *chunk_off = reinterpret_cast<int32_t *>(ws + lay.chunk_off);
    float *seg_out = reinterpret_cast<float *>(ws + lay.seg_out);
    float *seg_init = reinterpret_cast<float *>(ws + lay.seg_init);
    void *img = ws + lay.img;
    // summaries in the order the combine loads them (see kda_prefill.hip, CMB_ROWS)
    const int32_t cmb_fmt = bf16 ? 2 : 1;
    // eight-wave 128-column workgroups when a pass has fewer workgroups than
    // the GPU has compute units (bf16)
    const int64_t out_wgs = (int64_t)(lay.pieces > 0 ? lay.pieces : lay.max_segs) * num_heads;
    const int32_t narrow_out = bf16 && out_wgs <= kNumCUs ? 1 : 0;
    const int32_t narrow_sum = bf16 && (int64_t)lay.max_units * num_heads <= kNumCUs ? 1 : 0;
    // output segments and summary units (SEG_LAST: in a sequence's last segment), one launch
    int32_t *seq_order = reinterpret_cast<int32_t *>(ws + lay.seq_order);
    // and the chunk operands of every (chunk, head); one launch for up to 256 sequences
    hipError_t e = kda_launch_cp_plan_prep(bf16, q, k, g, beta, cu_seqlens, num_seqs, total_tokens, num_heads,
                                           lay.max_chunks, img, nullptr, seg_len, lay.max_segs, plan, seq_seg,
                                           chunk_off, sched, 0, 0, nullptr, lay.unit_len, lay.max_units, uplan,
                                           useq_seg, usched, seg_len, 1, seq_order, lay.pieces, lay.piece_len, s);
    if (e == hipSuccess)   // unit summaries (units before a sequence's last segment)
        e = kda_launch_chain(bf16, kCpSumBlock, v, nullptr, cu_seqlens, num_seqs, total_tokens, num_heads, dv, out,
                             nullptr, uplan, lay.max_units, 1, nullptr, seg_out, chunk_off, img, usched, nullptr,
                             nullptr, nullptr, nullptr, nullptr, 0, 0, cmb_fmt, narrow_sum, 0, kCpSumTail, 0, nullptr,
                             0, s);
    if (e == hipSuccess)   // entering state of every unit up to the start of a sequence's last segment
        e = kda_launch_cp_combine(initial_state, num_seqs, num_heads, dv, useq_seg, seg_out, seg_init, 0, uplan,
                                  seq_order, nullptr, 0, cmb_fmt, s);
    if (e == hipSuccess)   // outputs and final states, each segment from the entering state of its first unit
        e = kda_launch_chain(bf16, kCpBlock, v, initial_state, cu_seqlens, num_seqs, total_tokens, num_heads, dv, out,
                             final_state, plan, lay.max_segs, 0, seg_init, nullptr, chunk_off, img, sched, nullptr,
                             nullptr, nullptr, nullptr, lay.pieces > 0 ? nullptr : useq_seg, lay.unit_len,
                             lay.max_units, 0, narrow_out, 1, 0, lay.pieces, nullptr, 0, s);
    return e == hipSuccess ? KDA_OK : KDA_ERR_LAUNCH;
}

}  // namespace

kda_status kda_prefill_cp(const void *q, const void *k, const void *v, const float *g,
                          const float *beta, const float *initial_state, const int32_t *cu_seqlens,
                          int32_t num_seqs, int32_t total_tokens, int32_t num_heads, int32_t dk,
                          int32_t dv, kda_dtype dtype, void *out, float *final_state, int32_t seg_len,
                          void *workspace, size_t workspace_bytes, kda_stream_t stream)
{
    CpLayout lay;
    kda_status st = cp_check(q, k, v, g, beta, cu_seqlens, num_seqs, total_tokens, num_heads, dk, dv, dtype, out,
                             &seg_len, &lay);
    if (st != KDA_OK) return st;
    if (!workspace || !aligned(workspace, 256) || workspace_bytes < lay.total) return KDA_ERR_INVALID_ARG;
    if (validate_enabled() && num_seqs > 0)
        if (kda_status v = validate_cu(cu_seqlens, num_seqs, total_tokens, reinterpret_cast<hipStream_t>(stream)))
            return v;
    return cp_launch(q, k, v, g, beta, initial_state, cu_seqlens, num_seqs, total_tokens, num_heads, dv, dtype, out,
                     final_state, seg_len, lay, workspace, reinterpret_cast<hipStream_t>(stream));
}

kda_status kda_prefill_cp_noalloc(const void *q, const void *k, const void *v, const float *g,
                                  const float *beta, const float *initial_state, const int32_t *cu_seqlens,
                                  int32_t num_seqs, int32_t total_tokens, int32_t num_heads, int32_t dk,
                                  int32_t dv, kda_dtype dtype, void *out, float *final_state, int32_t seg_len,
                                  kda_stream_t stream)
{
    CpLayout lay;
    kda_status st = cp_check(q, k, v, g, beta, cu_seqlens, num_seqs, total_tokens, num_heads, dk, dv, dtype, out,
                             &seg_len, &lay);
    if (st != KDA_OK) return st;
    if (lay.total > (size_t)KDA_STATIC_SCRATCH_BYTES) return KDA_ERR_SCRATCH;
    void *ws = nullptr;
    size_t bytes = 0;
    if (kda_static_scratch(&ws, &bytes) != hipSuccess || !ws || bytes < lay.total) return KDA_ERR_LAUNCH;
    return cp_launch(q, k, v, g, beta, initial_state, cu_seqlens, num_seqs, total_tokens, num_heads, dv, dtype, out,
                     final_state, seg_len, lay, ws, reinterpret_cast<hipStream_t>(stream));
}

kda_status kda_decode_step(const void *q, const void *k, const void *v, const float *g,
                           const float *beta, float *state_inout, int32_t num_seqs,
                           int32_t num_heads, int32_t dk, int32_t dv, kda_dtype dtype, void *out,
                           kda_stream_t stream)
{
    kda_status st = check_common(q, k, v, g, beta, out, dk, dv, dtype);
    if (st == KDA_ERR_INVALID_ARG) return st;
    if (!state_inout || !aligned(state_inout, 16) || num_seqs < 0 || num_heads <= 0)
        return KDA_ERR_INVALID_ARG;
    if (st != KDA_OK) return st;
    const int64_t units = (int64_t)num_seqs * num_heads;
    if (units == 0) return KDA_OK;
    if (units > INT32_MAX) return KDA_ERR_INVALID_ARG;
    hipError_t e = kda_launch_decode(dtype == KDA_BF16 ? 1 : 0, q, k, v, g, beta, state_inout,
                                     num_seqs, num_heads, out, reinterpret_cast<hipStream_t>(stream));
    return e == hipSuccess ? KDA_OK : KDA_ERR_LAUNCH;
}

kda_status kda_decode_tokens(const void *q, const void *k, const void *v, const float *g,
                             const float *beta, const int32_t *cu_seqlens, const int32_t *num_tokens,
                             const float *state_in, float *state_out, int32_t num_seqs,
                             int32_t total_tokens, int32_t num_heads, int32_t dk, int32_t dv,
                             kda_dtype dtype, void *out, kda_stream_t stream)
{
    // out may be NULL (replay only): validate it only when given
    kda_status st = check_common(q, k, v, g, beta, out ? out : q, dk, dv, dtype);
    if (st == KDA_ERR_INVALID_ARG) return st;
    if (!cu_seqlens || !state_in || !aligned(state_in, 16) || (state_out && !aligned(state_out, 16)) ||
        num_seqs < 0 || total_tokens < 0 || num_heads <= 0)
        return KDA_ERR_INVALID_ARG;
    if (st != KDA_OK) return st;
    const int64_t units = (int64_t)num_seqs * num_heads;
    if (units == 0) return KDA_OK;
    if (units > INT32_MAX) return KDA_ERR_INVALID_ARG;
    if (validate_enabled())
        if (kda_status v = validate_cu(cu_seqlens, num_seqs, total_tokens, reinterpret_cast<hipStream_t>(stream)))
            return v;
    hipError_t e = kda_launch_decode_tokens(dtype == KDA_BF16 ? 1 : 0, q, k, v, g, beta, cu_seqlens, num_tokens,
                                           state_in, state_out, num_seqs, total_tokens, num_heads, out,
                                           reinterpret_cast<hipStream_t>(stream));
    return e == hipSuccess ? KDA_OK : KDA_ERR_LAUNCH;
}

// ---------------------------------------------------------------- backward
namespace {

struct BwdLayout {
    size_t plan, sched, seq_seg, chunk_off, img, gimg, snaps, gchunk, sscale, gscale, uw_u, uw_w, dx, fsum, bsum,
        seg_init, seg_dsend, hflag, total;
    int32_t max_chunks, max_segs, seg_len;
};

// Segment length of the backward, shared with the forward pipeline that
// stores the chunk-start states (so that a segment's gradient transition is
// the transpose of its forward transition): about 256 segments per head
// count, at least 256 tokens, a multiple of the chunk.
int32_t bwd_seg_len(int32_t T, int32_t H)
{
    int64_t len = (int64_t)T * H / 256;
    len = len < 256 ? 256 : (len > 65536 ? 65536 : len);
    return (int32_t)((len + kCpChunk - 1) / kCpChunk * kCpChunk);
}

// Workspace sections: the plan [max_segs][4] int32 (no segment marked last:
// the forward summaries cover every segment), its dispatch order [max_segs]
// and the first segment [N+1] and first chunk [N+1] of each sequence; the
// chunk images and the gradient images (same slots); forward states at chunk
// starts and state gradients at chunk ends [max_chunks][H][dk][dv] (fp32, or
// fp16 with column scales [max_chunks][H][dv] each for bf16 inputs); every
// chunk's U, W (forward) and dX (state gradient) [max_chunks][H][32][dv]; forward
// summaries [max_segs][H][dk (dv + 2 dk)] (S^0, M and M^T in the combine's
// fragment layout); gradient summaries [max_segs][H][dk][dv];
// entering states and entering gradients [max_segs][H][dk][dv] (the two
// strands of the pipeline run side by side, so each has its own; these three
// as accumulator tiles).
bool bwd_layout(int32_t N, int32_t T, int32_t H, int bf16, BwdLayout *lay)
{
    const int32_t seg_len = bwd_seg_len(T, H);
    const int64_t chunks = (int64_t)T / kCpChunk + 1 + N;
    const int64_t segs = (int64_t)T / seg_len + 1 + N;
    if (chunks > INT32_MAX / 4 || segs > INT32_MAX / 4) return false;
    const size_t S = (size_t)kHeadDim * kHeadDim;
    const size_t img = kda_chunk_image_bytes(bf16) * (size_t)chunks * H;
    lay->seg_len = seg_len;
    lay->max_chunks = (int32_t)chunks;
    lay->max_segs = (int32_t)segs;
    lay->plan = 0;
    lay->sched = align256(lay->plan + sizeof(int32_t) * 4 * (size_t)segs);
    lay->seq_seg = align256(lay->sched + sizeof(int32_t) * (size_t)segs);
    lay->chunk_off = align256(lay->seq_seg + sizeof(int32_t) * ((size_t)N + 1));
    lay->img = align256(lay->chunk_off + sizeof(int32_t) * ((size_t)N + 1));
    lay->gimg = align256(lay->img + img);
    lay->snaps = align256(lay->gimg + img);
    lay->gchunk = align256(lay->snaps + sizeof(float) * (size_t)chunks * H * S);
    lay->sscale = align256(lay->gchunk + sizeof(float) * (size_t)chunks * H * S);
    lay->gscale = align256(lay->sscale + sizeof(float) * (size_t)chunks * H * kHeadDim);
    lay->uw_u = align256(lay->gscale + sizeof(float) * (size_t)chunks * H * kHeadDim);
    lay->uw_w = align256(lay->uw_u + sizeof(float) * (size_t)chunks * H * kCpChunk * kHeadDim);
    lay->dx = align256(lay->uw_w + sizeof(float) * (size_t)chunks * H * kCpChunk * kHeadDim);
    lay->fsum = align256(lay->dx + sizeof(float) * (size_t)chunks * H * kCpChunk * kHeadDim);
    lay->bsum = align256(lay->fsum + sizeof(float) * (size_t)segs * H * 3 * S);
    lay->seg_init = align256(lay->bsum + sizeof(float) * (size_t)segs * H * S);
    lay->seg_dsend = align256(lay->seg_init + sizeof(float) * (size_t)segs * H * S);
    lay->hflag = align256(lay->seg_dsend + sizeof(float) * (size_t)segs * H * S);
    lay->total = align256(lay->hflag + sizeof(int32_t) * (size_t)segs * H);
    return true;
}

// A second stream per device for the backward: its two strands (states of
// the forward, gradients of the state) are chains of small launches that
// leave most compute units idle, so they run side by side -- forked from and
// joined back into the caller's stream with events, which also works under
// stream capture.  Created on first use (default priority, non-blocking),
// kept until the process ends; the enqueue sequence of one call holds the
// device's mutex, so calls from several host threads do not interleave their
// event records.  If creation fails, everything runs on the caller's stream.
struct SideStream {
    hipStream_t stream = nullptr;
    hipEvent_t ev[3] = {nullptr, nullptr, nullptr};
    bool ready = false;
    std::mutex use;
};
SideStream g_side[64];
std::mutex g_side_init;

SideStream *side_stream()
{
    int dev = -1;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return nullptr;
    SideStream &ss = g_side[dev];
    std::lock_guard<std::mutex> lk(g_side_init);
    if (!ss.ready) {
        bool ok = hipStreamCreateWithFlags(&ss.stream, hipStreamNonBlocking) == hipSuccess;
        for (int i = 0; i < 3 && ok; ++i) ok = hipEventCreateWithFlags(&ss.ev[i], hipEventDisableTiming) == hipSuccess;
        if (!ok) {
            for (int i = 0; i < 3; ++i)
                if (ss.ev[i]) (void)hipEventDestroy(ss.ev[i]), ss.ev[i] = nullptr;
            if (ss.stream) (void)hipStreamDestroy(ss.stream), ss.stream = nullptr;
            (void)hipGetLastError();
            return nullptr;
        }
        ss.ready = true;
    }
    return &ss;
}

}  // namespace

size_t kda_backward_workspace_size(int32_t num_seqs, int32_t total_tokens, int32_t num_heads, int32_t dk, int32_t dv,
                                   kda_dtype dtype)
{
    if (num_seqs < 0 || total_tokens < 0 || num_heads <= 0 || dk != kHeadDim || dv != kHeadDim) return 0;
    if (dtype != KDA_F32 && dtype != KDA_BF16) return 0;
    BwdLayout lay;
    if (!bwd_layout(num_seqs, total_tokens, num_heads, dtype == KDA_BF16, &lay)) return 0;
    return lay.total;
}

kda_status kda_backward(const void *q, const void *k, const void *v, const float *g, const float *beta,
                        const float *initial_state, const int32_t *cu_seqlens, int32_t num_seqs,
                        int32_t total_tokens, int32_t num_heads, int32_t dk, int32_t dv, kda_dtype dtype,
                        const void *dout, const float *dfinal, float *dq, float *dk_out, float *dv_out,
                        float *dg, float *dbeta, float *dinit, void *workspace, size_t workspace_bytes,
                        kda_stream_t stream)
{
    kda_status st = check_common(q, k, v, g, beta, dout, dk, dv, dtype);
    if (st == KDA_ERR_INVALID_ARG) return st;
    if (!cu_seqlens || num_seqs < 0 || total_tokens < 0 || num_heads <= 0) return KDA_ERR_INVALID_ARG;
    if (!dq || !dk_out || !dv_out || !dg || !dbeta) return KDA_ERR_INVALID_ARG;
    if (!aligned(dq, 16) || !aligned(dk_out, 16) || !aligned(dv_out, 16) || !aligned(dg, 16) ||
        !aligned(dbeta, 4) || (dfinal && !aligned(dfinal, 16)) || (dinit && !aligned(dinit, 16)) ||
        (initial_state && !aligned(initial_state, 16)))
        return KDA_ERR_INVALID_ARG;
    if (st != KDA_OK) return st;
    BwdLayout lay;
    if (!bwd_layout(num_seqs, total_tokens, num_heads, dtype == KDA_BF16, &lay)) return KDA_ERR_INVALID_ARG;
    if (!workspace || !aligned(workspace, 256) || workspace_bytes < lay.total) return KDA_ERR_INVALID_ARG;
    const int64_t units = (int64_t)num_seqs * num_heads;
    if (units == 0) return KDA_OK;
    if ((int64_t)lay.max_segs * num_heads * ((dv + dk) / 16) > INT32_MAX ||
        (int64_t)lay.max_chunks * num_heads > INT32_MAX)
        return KDA_ERR_INVALID_ARG;
    if (validate_enabled())
        if (kda_status v = validate_cu(cu_seqlens, num_seqs, total_tokens, reinterpret_cast<hipStream_t>(stream)))
            return v;
    const int bf16 = dtype == KDA_BF16 ? 1 : 0;
    char *ws = static_cast<char *>(workspace);
    int32_t *plan = reinterpret_cast<int32_t *>(ws + lay.plan);
    int32_t *sched = reinterpret_cast<int32_t *>(ws + lay.sched);
    int32_t *seq_seg = reinterpret_cast<int32_t *>(ws + lay.seq_seg);
    int32_t *chunk_off = reinterpret_cast<int32_t *>(ws + lay.chunk_off);
    void *snaps = ws + lay.snaps;
    float *fsum = reinterpret_cast<float *>(ws + lay.fsum);
    float *bsum = reinterpret_cast<float *>(ws + lay.bsum);
    float *seg_init = reinterpret_cast<float *>(ws + lay.seg_init);
    float *seg_dsend = reinterpret_cast<float *>(ws + lay.seg_dsend);
    void *img = ws + lay.img;
    void *gimg = ws + lay.gimg;
    void *gchunk = ws + lay.gchunk;
    float *sscale = reinterpret_cast<float *>(ws + lay.sscale);
    float *gscale = reinterpret_cast<float *>(ws + lay.gscale);
    float *uw_u = reinterpret_cast<float *>(ws + lay.uw_u);
    float *uw_w = reinterpret_cast<float *>(ws + lay.uw_w);
    float *dxc = reinterpret_cast<float *>(ws + lay.dx);
    hipStream_t s = reinterpret_cast<hipStream_t>(stream);
    // Two strands after the chunk operands, on the caller's stream s and the
    // side stream s2 (s itself when there is none):
    //   s:  forward summaries -> forward combine -> forward states at chunk starts
    //   s2: gradient summaries -> (forward summaries done) reverse combine ->
    //       state gradients at chunk ends
    // (with the head walk below, both summary passes run on s first and s2
    // starts at the reverse combine); then, on s once both strands are done,
    // the per-chunk gradients.
    SideStream *ss = side_stream();
    std::unique_lock<std::mutex> lk;
    if (ss) lk = std::unique_lock<std::mutex>(ss->use);
    hipStream_t s2 = ss ? ss->stream : s;
    auto fork = [&](int i, hipStream_t from, hipStream_t to) -> hipError_t {
        if (!ss) return hipSuccess;
        hipError_t r = hipEventRecord(ss->ev[i], from);
        return r == hipSuccess ? hipStreamWaitEvent(to, ss->ev[i], 0) : r;
    };
    // segments and chunk numbering (no segment is marked last, so the forward
    // summaries include every segment's transition), and the chunk operands of
    // every (chunk, head): the forward image and the transposed one of the
    // gradient chain; one launch for up to 256 sequences
    hipError_t e = kda_launch_cp_plan_prep(bf16, q, k, g, beta, cu_seqlens, num_seqs, total_tokens, num_heads,
                                           lay.max_chunks, img, gimg, lay.seg_len, lay.max_segs, plan, seq_seg,
                                           chunk_off, sched, -1, 0, nullptr, 0, 0, nullptr, nullptr, nullptr, 0, 0,
                                           nullptr, 0, 0, s);
    // summaries in the combine's operand order, with M^T for the reverse
    // walk; summaries of gradients, entering states and entering gradients as
    // accumulator tiles (see kda_prefill.hip, CMB_ROWS)
    const int32_t cmb_fmt = (bf16 ? 2 : 1) | 4;
    // Head walk (16-bit inputs, segments of more than kCpSumTail chunks): the
    // forward summaries flag every segment whose transition over its first
    // kCpSumTail chunks is exactly zero, and the gradient summaries of those
    // segments walk only those chunks.  The gradient summaries then follow the
    // forward summaries on the caller's stream, ahead of the state pass, which
    // would otherwise hold the compute units they wait for; without the head
    // walk the two summary passes run side by side.
    const bool head = bf16 && lay.seg_len / kCpChunk > kCpSumTail;
    int32_t *hflag = head ? reinterpret_cast<int32_t *>(ws + lay.hflag) : nullptr;
    const int32_t sum_head = head ? kCpSumTail : 0;
    auto fwd_summaries = [&](hipStream_t st) {   // forward summaries [S^0 | M | M^T] of every segment
        return kda_launch_chain(bf16, kCpSumBlock, v, nullptr, cu_seqlens, num_seqs, total_tokens, num_heads, dv,
                                nullptr, nullptr, plan, lay.max_segs, 1, nullptr, fsum, chunk_off, img, sched,
                                nullptr, nullptr, nullptr, nullptr, nullptr, 0, 0, cmb_fmt, 0, 0, 0, 0, hflag,
                                sum_head, st);
    };
    auto grad_summaries = [&](hipStream_t st) {  // gradient summaries G^0 of every segment but a sequence's first
        return kda_launch_grad_chain(bf16, 1, dout, cu_seqlens, num_seqs, total_tokens, num_heads, plan,
                                     lay.max_segs, sched, chunk_off, gimg, nullptr, nullptr, nullptr, nullptr, bsum,
                                     nullptr, 1, hflag, sum_head, st);
    };
    bool forked = false;
    if (head) {
        if (e == hipSuccess) e = fwd_summaries(s);
        if (e == hipSuccess) e = grad_summaries(s);
        if (e == hipSuccess) {
            e = fork(0, s, s2);
            forked = e == hipSuccess;
        }
    } else {
        if (e == hipSuccess) {
            e = fork(0, s, s2);
            forked = e == hipSuccess;
        }
        if (e == hipSuccess) e = grad_summaries(s2);
        if (e == hipSuccess) e = fwd_summaries(s);
        if (e == hipSuccess) e = fork(1, s, s2);
    }
    if (e == hipSuccess)   // s2: the gradient entering every segment at its end, with R_s = M_s^T
        e = kda_launch_cp_combine(dfinal, num_seqs, num_heads, dv, seq_seg, bsum, seg_dsend, 1, nullptr, nullptr,
                                  fsum, 1, cmb_fmt, s2);
    if (e == hipSuccess)   // s2: the gradient at every chunk end, every chunk's dX, and d(initial state)
        e = kda_launch_grad_chain(bf16, 0, dout, cu_seqlens, num_seqs, total_tokens, num_heads, plan, lay.max_segs,
                                  sched, chunk_off, gimg, seg_dsend, gchunk, gscale, dinit, nullptr, dxc, 1, nullptr,
                                  0, s2);
    if (e == hipSuccess)   // s: the state entering every segment
        e = kda_launch_cp_combine(initial_state, num_seqs, num_heads, dv, seq_seg, fsum, seg_init, 0, nullptr,
                                  nullptr, nullptr, 0, cmb_fmt, s);
    if (e == hipSuccess)   // s: the state at every chunk start, and every chunk's U and W
        e = kda_launch_chain(bf16, kCpBlock, v, initial_state, cu_seqlens, num_seqs, total_tokens, num_heads, dv,
                             nullptr, nullptr, plan, lay.max_segs, 0, seg_init, nullptr, chunk_off, img, sched,
                             snaps, sscale, uw_u, uw_w, nullptr, 0, 0, 0, 0, 1, 0, 0, nullptr, 0, s);
    if (forked) {          // join: s waits for s2 (also after a failed launch)
        const hipError_t j = fork(2, s2, s);
        if (e == hipSuccess) e = j;
    }
    if (e == hipSuccess)   // every chunk's gradients of q, k, v, g and beta
        e = kda_launch_bwd_chunk(bf16, q, k, g, beta, dout, cu_seqlens, chunk_off, lay.max_chunks, snaps, sscale,
                                 gchunk, gscale, uw_u, uw_w, dxc, num_seqs, total_tokens, num_heads, dq, dk_out,
                                 dv_out, dg, dbeta, s);
    return e == hipSuccess ? KDA_OK : KDA_ERR_LAUNCH;
}

const char *kda_status_string(kda_status status)
{
    switch (status) {
    case KDA_OK: return "KDA_OK: success";
    case KDA_ERR_INVALID_ARG: return "KDA_ERR_INVALID_ARG: invalid argument (null, negative, misaligned or bad dtype)";
    case KDA_ERR_UNSUPPORTED: return "KDA_ERR_UNSUPPORTED: valid but unsupported configuration (v1: dk = dv = 128)";
    case KDA_ERR_LAUNCH: return "KDA_ERR_LAUNCH: HIP kernel launch failed";
    case KDA_ERR_SCRATCH:
        return "KDA_ERR_SCRATCH: the problem needs more workspace than the library's static device scratch "
               "(KDA_STATIC_SCRATCH_BYTES) holds; use kda_prefill_cp with a caller-owned workspace";
    }
    return "unknown kda_status";
}

int32_t kda_version(void) { return 100; }

}  // extern "C"
