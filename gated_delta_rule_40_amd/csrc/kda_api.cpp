// kda_api.cpp -- host side of the libkda C ABI (declared in include/kda.h).
//
// Validates every argument before touching HIP, picks the kernel tiling and
// launches on the caller's stream.  No device memory is allocated, no stream
// is synchronised and no mutable state is shared between calls.
#include <hip/hip_runtime.h>

#include <cstdint>

#include "kda.h"

extern "C" hipError_t kda_launch_prefill(int bf16, int chunk, int dv_block, const void *q,
                                         const void *k, const void *v, const float *g,
                                         const float *beta, const float *init, const int32_t *cu,
                                         int32_t N, int32_t T_tot, int32_t H, int32_t dv,
                                         void *out, float *fin, float *snap, int32_t snap_every,
                                         int32_t max_snaps, const int32_t *snap_chunk_off, hipStream_t stream);
extern "C" hipError_t kda_launch_cp_plan(const int32_t *cu, int32_t N, int32_t T_tot, int32_t seg_len,
                                         int32_t max_segs, int32_t *plan, int32_t *seq_seg, int32_t chunk,
                                         int32_t max_chunks, int32_t *chunk_off, int32_t *sched,
                                         int32_t last_len, int32_t skip_last, int32_t *seq_order,
                                         int32_t seg_len2, int32_t max_segs2, int32_t *plan2, int32_t *seq_seg2,
                                         int32_t *sched2, int32_t last_len2, int32_t skip_last2,
                                         int32_t *seq_order2, hipStream_t stream);
extern "C" hipError_t kda_launch_chunk_prep(int bf16, const void *q, const void *k, const float *g,
                                            const float *beta, const int32_t *cu, int32_t N, int32_t T_tot,
                                            int32_t H, const int32_t *chunk_off, int64_t max_chunks, void *img,
                                            hipStream_t stream);
extern "C" hipError_t kda_launch_chain(int bf16, int dv_block, const void *v, const float *init, const int32_t *cu, int32_t N,
                                       int32_t T_tot, int32_t H, int32_t dv, void *out, float *fin,
                                       const int32_t *plan, int32_t num_segs, int32_t mode, const float *seg_init,
                                       float *seg_out, const int32_t *chunk_off, const void *img,
                                       const int32_t *sched, float *snap, const int32_t *init_seq_seg,
                                       int32_t init_unit, int32_t init_units, hipStream_t stream);
extern "C" size_t kda_chunk_image_bytes(int bf16);
extern "C" hipError_t kda_launch_backward_summary(int bf16, const void *q, const void *k, const float *g,
                                                  const float *beta, const void *dout, const int32_t *plan,
                                                  int32_t num_segs, int32_t T_tot, int32_t H, int32_t ncols,
                                                  float *seg_out, hipStream_t stream);
extern "C" size_t kda_backward_scratch_floats_per_wg();
extern "C" int32_t kda_backward_max_wgs();
extern "C" int32_t kda_backward_num_blocks();
extern "C" hipError_t kda_launch_backward(int bf16, const void *q, const void *k, const void *v, const float *g,
                                          const float *beta, const float *init, const int32_t *cu,
                                          const int32_t *chunk_off, const float *snaps, const void *dout,
                                          const int32_t *plan, int32_t num_segs, const float *seg_dsend,
                                          int32_t N, int32_t T_tot, int32_t H, float *scratch,
                                          float *part_vec, float *part_beta, float *dq, float *dk, float *dv,
                                          float *dg, float *dbeta, float *dinit, hipStream_t stream);
extern "C" hipError_t kda_launch_decode_tokens(int bf16, const void *q, const void *k, const void *v,
                                               const float *g, const float *beta, const int32_t *cu,
                                               const int32_t *num_tokens, const float *state_in,
                                               float *state_out, int32_t N, int32_t T_tot, int32_t H, void *out,
                                               hipStream_t stream);
extern "C" hipError_t kda_launch_cp_combine(const float *init, int32_t N, int32_t H, int32_t dv,
                                            const int32_t *seq_seg, const float *seg_out, float *seg_init,
                                            int32_t reverse, const int32_t *plan, const int32_t *seq_order,
                                            const float *m_src, int32_t m_trans, hipStream_t stream);
extern "C" hipError_t kda_launch_decode(int bf16, const void *q, const void *k, const void *v,
                                        const float *g, const float *beta, float *state,
                                        int32_t N, int32_t H, void *out, hipStream_t stream);

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

struct CpLayout {
    size_t plan, sched, seq_seg, uplan, usched, useq_seg, seq_order, chunk_off, seg_out, seg_init, img, total;
    int32_t max_segs, max_units, unit_len, max_chunks;
};

size_t align256(size_t x) { return (x + 255) & ~size_t(255); }

// Summary units: when there are at least as many (segment, head) pairs as
// compute units (T / seg_len * H >= 256), output segments (seg_len tokens) are
// cut into up to four units for the summary pass and the combine, so that the
// summary pass, one workgroup per (unit, head) at one per compute unit, is
// made of many short pieces that pack the GPU evenly; the output pass still
// runs whole segments, from the entering state of their first unit.  Below
// that the summary pass is a single round anyway, and more units would only
// lengthen the combine's chain.  The unit length divides seg_len and is a
// multiple of the chunk.
int32_t cp_unit_len(int32_t seg_len, int32_t T, int32_t H)
{
    const int32_t m = seg_len / kCpChunk;
    if ((int64_t)T / seg_len * H < 256) return seg_len;
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
bool cp_layout(int32_t N, int32_t T, int32_t H, int32_t dk, int32_t dv, int bf16, int32_t seg_len, CpLayout *lay)
{
    const int32_t unit = cp_unit_len(seg_len, T, H);
    const int64_t segs = (int64_t)T / seg_len + 1 + N;
    const int64_t units = (int64_t)T / unit + 1 + N;
    const int64_t chunks = (int64_t)T / kCpChunk + 1 + N;
    if (units > INT32_MAX / 4 || chunks > INT32_MAX / 4) return false;
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

// Default segment length: about 512 (segment, head) pairs (two output-pass
// workgroups per compute unit), at least 256 tokens (8 chunks: shorter
// segments add more combine steps than they take off a workgroup's walk;
// 4,096 tokens x 8 heads: 0.132 ms at 256, 0.145 ms at 512, 0.41 ms at 128)
// and at most 65,536.
int32_t cp_default_seg_len(int32_t T, int32_t H)
{
    int64_t len = (int64_t)T * H / 512;
    len = len < 256 ? 256 : (len > 65536 ? 65536 : len);
    return (int32_t)((len + kCpChunk - 1) / kCpChunk * kCpChunk);
}

}  // namespace

size_t kda_prefill_cp_workspace_size(int32_t num_seqs, int32_t total_tokens, int32_t num_heads,
                                     int32_t dk, int32_t dv, kda_dtype dtype, int32_t seg_len)
{
    if (num_seqs < 0 || total_tokens < 0 || num_heads <= 0 || dk != kHeadDim || dv != kHeadDim) return 0;
    if (dtype != KDA_F32 && dtype != KDA_BF16) return 0;
    if (seg_len == 0) seg_len = cp_default_seg_len(total_tokens, num_heads);
    if (seg_len < kCpChunk || seg_len % kCpChunk) return 0;
    CpLayout lay;
    if (!cp_layout(num_seqs, total_tokens, num_heads, dk, dv, dtype == KDA_BF16, seg_len, &lay)) return 0;
    return lay.total;
}

kda_status kda_prefill_cp(const void *q, const void *k, const void *v, const float *g,
                          const float *beta, const float *initial_state, const int32_t *cu_seqlens,
                          int32_t num_seqs, int32_t total_tokens, int32_t num_heads, int32_t dk,
                          int32_t dv, kda_dtype dtype, void *out, float *final_state, int32_t seg_len,
                          void *workspace, size_t workspace_bytes, kda_stream_t stream)
{
    kda_status st = check_common(q, k, v, g, beta, out, dk, dv, dtype);
    if (st == KDA_ERR_INVALID_ARG) return st;
    if (!cu_seqlens || num_seqs < 0 || total_tokens < 0 || num_heads <= 0 || seg_len < 0)
        return KDA_ERR_INVALID_ARG;
    if (st != KDA_OK) return st;
    if (seg_len == 0) seg_len = cp_default_seg_len(total_tokens, num_heads);
    if (seg_len < kCpChunk || seg_len % kCpChunk) return KDA_ERR_UNSUPPORTED;
    const int bf16 = dtype == KDA_BF16 ? 1 : 0;
    CpLayout lay;
    if (!cp_layout(num_seqs, total_tokens, num_heads, dk, dv, bf16, seg_len, &lay)) return KDA_ERR_INVALID_ARG;
    if (!workspace || !aligned(workspace, 256) || workspace_bytes < lay.total) return KDA_ERR_INVALID_ARG;
    if ((int64_t)lay.max_units * num_heads * ((dv + dk) / 16) > INT32_MAX) return KDA_ERR_INVALID_ARG;
    if ((int64_t)lay.max_chunks * num_heads > INT32_MAX) return KDA_ERR_INVALID_ARG;
    if (num_seqs == 0) return KDA_OK;
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
    hipStream_t s = reinterpret_cast<hipStream_t>(stream);
    // output segments and summary units (SEG_LAST: in a sequence's last segment), one launch
    int32_t *seq_order = reinterpret_cast<int32_t *>(ws + lay.seq_order);
    hipError_t e = kda_launch_cp_plan(cu_seqlens, num_seqs, total_tokens, seg_len, lay.max_segs, plan, seq_seg,
                                      kCpChunk, lay.max_chunks, chunk_off, sched, 0, 0, nullptr, lay.unit_len,
                                      lay.max_units, uplan, useq_seg, usched, seg_len, 1, seq_order, s);
    if (e == hipSuccess)   // chunk operands of every (chunk, head)
        e = kda_launch_chunk_prep(bf16, q, k, g, beta, cu_seqlens, num_seqs, total_tokens, num_heads, chunk_off,
                                  lay.max_chunks, img, s);
    if (e == hipSuccess)   // unit summaries (units before a sequence's last segment)
        e = kda_launch_chain(bf16, kCpSumBlock, v, nullptr, cu_seqlens, num_seqs, total_tokens, num_heads, dv, out,
                             nullptr, uplan, lay.max_units, 1, nullptr, seg_out, chunk_off, img, usched, nullptr,
                             nullptr, 0, 0, s);
    if (e == hipSuccess)   // entering state of every unit up to the start of a sequence's last segment
        e = kda_launch_cp_combine(initial_state, num_seqs, num_heads, dv, useq_seg, seg_out, seg_init, 0, uplan,
                                  seq_order, nullptr, 0, s);
    if (e == hipSuccess)   // outputs and final states, each segment from the entering state of its first unit
        e = kda_launch_chain(bf16, kCpBlock, v, initial_state, cu_seqlens, num_seqs, total_tokens, num_heads, dv, out,
                             final_state, plan, lay.max_segs, 0, seg_init, nullptr, chunk_off, img, sched, nullptr,
                             useq_seg, lay.unit_len, lay.max_units, s);
    return e == hipSuccess ? KDA_OK : KDA_ERR_LAUNCH;
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
    hipError_t e = kda_launch_decode_tokens(dtype == KDA_BF16 ? 1 : 0, q, k, v, g, beta, cu_seqlens, num_tokens,
                                           state_in, state_out, num_seqs, total_tokens, num_heads, out,
                                           reinterpret_cast<hipStream_t>(stream));
    return e == hipSuccess ? KDA_OK : KDA_ERR_LAUNCH;
}

// ---------------------------------------------------------------- backward
namespace {

struct BwdLayout {
    size_t plan, sched, seq_seg, chunk_off, img, snaps, fsum, bsum, seg_dsend, scratch, part_vec, part_beta, total;
    int32_t max_chunks, max_segs, seg_len;
};

// Segment length of the backward, shared with the forward pipeline that
// stores the chunk-start states (so that a segment's gradient transition is
// the transpose of its forward transition): about 256 segments per head
// count (about 1,024 work items of (segment, head, 32 columns), two per
// workgroup of the main pass), at least 256 tokens, a multiple of the chunk.
int32_t bwd_seg_len(int32_t T, int32_t H)
{
    int64_t len = (int64_t)T * H / 256;
    len = len < 256 ? 256 : (len > 65536 ? 65536 : len);
    return (int32_t)((len + kCpChunk - 1) / kCpChunk * kCpChunk);
}

// Workspace sections: the plan [max_segs][4] int32 (no segment marked last:
// the forward summaries cover every segment), its dispatch order [max_segs]
// and the first segment [N+1] and first chunk [N+1] of each sequence; the
// chunk images; forward states at chunk starts [max_chunks][H][dk][dv];
// forward summaries [max_segs][H][dk][dv + dk]; gradient summaries
// [max_segs][H][dk][dv]; entering states, then entering gradients
// [max_segs][H][dk][dv]; the main pass's per-workgroup scratch; the partial
// row sums of dq, dk, dg and dbeta.
bool bwd_layout(int32_t N, int32_t T, int32_t H, int bf16, BwdLayout *lay)
{
    const int32_t seg_len = bwd_seg_len(T, H);
    const int64_t chunks = (int64_t)T / kCpChunk + 1 + N;
    const int64_t segs = (int64_t)T / seg_len + 1 + N;
    if (chunks > INT32_MAX / 4 || segs > INT32_MAX / 4) return false;
    const size_t S = (size_t)kHeadDim * kHeadDim;
    const size_t rows = (size_t)T * H;
    const size_t nblk = (size_t)kda_backward_num_blocks();
    const int64_t items = segs * H * (int64_t)nblk;
    const size_t wgs = (size_t)(items < kda_backward_max_wgs() ? items : kda_backward_max_wgs());
    lay->seg_len = seg_len;
    lay->max_chunks = (int32_t)chunks;
    lay->max_segs = (int32_t)segs;
    lay->plan = 0;
    lay->sched = align256(lay->plan + sizeof(int32_t) * 4 * (size_t)segs);
    lay->seq_seg = align256(lay->sched + sizeof(int32_t) * (size_t)segs);
    lay->chunk_off = align256(lay->seq_seg + sizeof(int32_t) * ((size_t)N + 1));
    lay->img = align256(lay->chunk_off + sizeof(int32_t) * ((size_t)N + 1));
    lay->snaps = align256(lay->img + kda_chunk_image_bytes(bf16) * (size_t)chunks * H);
    lay->fsum = align256(lay->snaps + sizeof(float) * (size_t)chunks * H * S);
    lay->bsum = align256(lay->fsum + sizeof(float) * (size_t)segs * H * 2 * S);
    lay->seg_dsend = align256(lay->bsum + sizeof(float) * (size_t)segs * H * S);
    lay->scratch = align256(lay->seg_dsend + sizeof(float) * (size_t)segs * H * S);
    lay->part_vec = align256(lay->scratch + sizeof(float) * wgs * kda_backward_scratch_floats_per_wg());
    lay->part_beta = align256(lay->part_vec + sizeof(float) * nblk * 3 * rows * kHeadDim);
    lay->total = align256(lay->part_beta + sizeof(float) * nblk * rows);
    return true;
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
    const int bf16 = dtype == KDA_BF16 ? 1 : 0;
    char *ws = static_cast<char *>(workspace);
    int32_t *plan = reinterpret_cast<int32_t *>(ws + lay.plan);
    int32_t *sched = reinterpret_cast<int32_t *>(ws + lay.sched);
    int32_t *seq_seg = reinterpret_cast<int32_t *>(ws + lay.seq_seg);
    int32_t *chunk_off = reinterpret_cast<int32_t *>(ws + lay.chunk_off);
    float *snaps = reinterpret_cast<float *>(ws + lay.snaps);
    float *fsum = reinterpret_cast<float *>(ws + lay.fsum);
    float *bsum = reinterpret_cast<float *>(ws + lay.bsum);
    float *seg_dsend = reinterpret_cast<float *>(ws + lay.seg_dsend);
    void *img = ws + lay.img;
    hipStream_t s = reinterpret_cast<hipStream_t>(stream);
    // segments and chunk numbering; no segment is marked last, so the forward
    // summaries include every segment's transition
    hipError_t e = kda_launch_cp_plan(cu_seqlens, num_seqs, total_tokens, lay.seg_len, lay.max_segs, plan, seq_seg,
                                      kCpChunk, lay.max_chunks, chunk_off, sched, -1, 0, nullptr, 0, 0, nullptr,
                                      nullptr, nullptr, 0, 0, nullptr, s);
    // forward: the state at every chunk start, by the context-parallel
    // pipeline with state stores and no outputs
    if (e == hipSuccess)
        e = kda_launch_chunk_prep(bf16, q, k, g, beta, cu_seqlens, num_seqs, total_tokens, num_heads, chunk_off,
                                  lay.max_chunks, img, s);
    if (e == hipSuccess)
        e = kda_launch_chain(bf16, kCpSumBlock, v, nullptr, cu_seqlens, num_seqs, total_tokens, num_heads, dv,
                             nullptr, nullptr, plan, lay.max_segs, 1, nullptr, fsum, chunk_off, img, sched,
                             nullptr, nullptr, 0, 0, s);
    if (e == hipSuccess)
        e = kda_launch_cp_combine(initial_state, num_seqs, num_heads, dv, seq_seg, fsum, seg_dsend, 0, nullptr,
                                  nullptr, nullptr, 0, s);
    if (e == hipSuccess)
        e = kda_launch_chain(bf16, kCpBlock, v, initial_state, cu_seqlens, num_seqs, total_tokens, num_heads, dv,
                             nullptr, nullptr, plan, lay.max_segs, 0, seg_dsend, nullptr, chunk_off, img, sched,
                             snaps, nullptr, 0, 0, s);
    if (e == hipSuccess)   // gradient summaries G^0 of every segment but a sequence's first
        e = kda_launch_backward_summary(bf16, q, k, g, beta, dout, plan, lay.max_segs, total_tokens, num_heads,
                                        dk, bsum, s);
    if (e == hipSuccess)   // the gradient entering every segment at its end, with R_s = M_s^T
        e = kda_launch_cp_combine(dfinal, num_seqs, num_heads, dv, seq_seg, bsum, seg_dsend, 1, nullptr, nullptr,
                                  fsum, 1, s);
    if (e == hipSuccess)
        e = kda_launch_backward(bf16, q, k, v, g, beta, initial_state, cu_seqlens, chunk_off, snaps, dout, plan,
                                lay.max_segs, seg_dsend, num_seqs, total_tokens, num_heads,
                                reinterpret_cast<float *>(ws + lay.scratch),
                                reinterpret_cast<float *>(ws + lay.part_vec),
                                reinterpret_cast<float *>(ws + lay.part_beta), dq, dk_out, dv_out, dg, dbeta, dinit,
                                s);
    return e == hipSuccess ? KDA_OK : KDA_ERR_LAUNCH;
}

const char *kda_status_string(kda_status status)
{
    switch (status) {
    case KDA_OK: return "KDA_OK: success";
    case KDA_ERR_INVALID_ARG: return "KDA_ERR_INVALID_ARG: invalid argument (null, negative, misaligned or bad dtype)";
    case KDA_ERR_UNSUPPORTED: return "KDA_ERR_UNSUPPORTED: valid but unsupported configuration (v1: dk = dv = 128)";
    case KDA_ERR_LAUNCH: return "KDA_ERR_LAUNCH: HIP kernel launch failed";
    }
    return "unknown kda_status";
}

int32_t kda_version(void) { return 100; }

}  // extern "C"
