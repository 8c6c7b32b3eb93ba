// Host side of librfw_atf.so: argument checks, the fp64 window table, the
// closed-form dropped-term count, the decode split planner and the C entry
// points declared in include/atf.h.
//
// Method: source page "ATFlash: RoPE-Frequenzen kuerzen Attention-Arbeit um
// bis zu 57 Prozent" (sudo-ai.de), section "Was ATFlash anders macht" (each
// rotary pair is cut beyond a distance proportional to its wavelength, the
// slow pairs keep far keys reachable) and section "Die Zahlen - und ihre
// Grenze" (prefill and decode keep the online softmax unchanged).

#include "../../include/atf.h"
#include "atf_internal.h"

#include <algorithm>
#include <cmath>
#include <cstdint>
#include <cstring>
#include <vector>

static_assert((size_t)ATF_NOALLOC_SCRATCH_BYTES == atf::kNoAllocScratchBytes, "scratch size");

using namespace atf;

namespace {

constexpr double kTwoPi = 6.283185307179586476925286766559;
constexpr int64_t kInf64 = INT64_MAX;
constexpr size_t kHeaderBytes = 256;  // workspace head: the dropped-term counter

// W_p = ceil(alpha * lambda_p), lambda_p = 2 pi base^(2p/d); the slowest pair
// and every pair at alpha = inf are uncut.  fp64 throughout: alpha*lambda_p
// sits at least ~3e-3 from an integer at every benchmarked setting, far
// beyond fp64 rounding, so the ceiling is stable.
void window_table(int d, double base, double alpha, int64_t *W) {
    const int P = d / 2;
    const double log_base = std::log(base);
    for (int p = 0; p < P; ++p) {
        if (p == P - 1 || std::isinf(alpha)) {
            W[p] = kInf64;
            continue;
        }
        const double lambda = kTwoPi * std::exp(log_base * (2.0 * p / d));
        const double x = std::ceil(alpha * lambda);
        W[p] = (x >= 9.0e18) ? kInf64 : (int64_t)x;
    }
}

// rotary angle step of pair p: base^(-2p/d)
void theta_table(int d, double base, double *theta) {
    const int P = d / 2;
    const double log_base = std::log(base);
    for (int p = 0; p < kMaxPairs; ++p) theta[p] = (p < P) ? std::exp(-log_base * (2.0 * p / d)) : 0.0;
}

// Windows as the kernels see them: int32, kWindowInf for "never cut".  Every
// distance a kernel meets is < 2^31 - 1, so clamping changes no decision.
void window_table_i32(int d, double base, double alpha, int *Wi) {
    int64_t W[kMaxPairs];
    window_table(d, base, alpha, W);
    for (int p = 0; p < kMaxPairs; ++p) {
        if (p >= d / 2 || W[p] >= (int64_t)kWindowInf) Wi[p] = kWindowInf;
        else Wi[p] = (int)W[p];
    }
}

bool aligned16(const void *p) { return p != nullptr && ((uintptr_t)p & 15u) == 0; }

// Head dims with compiled kernels.
bool supported_d(int32_t d) { return d == 64 || d == 128 || d == 256; }

atf_status check_shape(int32_t B, int32_t Hq, int32_t Hkv, int64_t S, int32_t d, double base,
                       double alpha, int32_t causal, int64_t pos0, atf_dtype dtype) {
    if (B < 1 || Hq < 1 || Hkv < 1 || S < 1) return ATF_ERR_INVALID_ARG;
    if (Hq % Hkv != 0) return ATF_ERR_INVALID_ARG;
    if (d < 2 || (d & 1)) return ATF_ERR_INVALID_ARG;
    if (!std::isfinite(base) || !(base > 1.0)) return ATF_ERR_INVALID_ARG;
    if (std::isnan(alpha) || !(alpha > 0.0)) return ATF_ERR_INVALID_ARG;
    if (dtype != ATF_F32 && dtype != ATF_BF16) return ATF_ERR_INVALID_ARG;
    if (causal != 0 && causal != 1) return ATF_ERR_INVALID_ARG;
    if (pos0 < 0 || pos0 + S + 1 >= (int64_t)INT32_MAX) return ATF_ERR_INVALID_ARG;
    if (!supported_d(d)) return ATF_ERR_UNSUPPORTED;
    if (Hq / Hkv > 64) return ATF_ERR_UNSUPPORTED;
    return ATF_OK;
}

bool bad_layout(int32_t layout) { return layout != ATF_ROPE_NEOX && layout != ATF_ROPE_GPTJ; }

size_t prefill_ws_bytes(int32_t B, int32_t Hkv, int64_t S, int32_t d, atf_dtype dtype) {
    if (dtype == ATF_F32) return kHeaderBytes;
    const size_t per = (size_t)B * Hkv * (size_t)padded_keys(S) * d * 2;  // bf16
    return kHeaderBytes + 2 * per;  // rotated keys + transposed values
}

// bf16 prefill work items.  Unpacked: a query tile of 8 waves' rows of one
// head (32 rows per wave; 16 on the 16x16x32 kernel, which runs d = 256).
// Head packed: one wave's rows of up to 8 heads sharing a kv head, so a short
// chunk does not run mostly empty tiles (a 16-query chunk fills 1/16 of a
// 256-row tile).  Packed when it runs fewer wave rows (its idle waves
// included).  A d = 128 chunk of at most 16 queries runs packed on the
// 16x16x32 kernel (narrow), whose 16-query waves carry no empty rows there.
struct PrefillPlan {
    int hpack, n_qtiles, group;  // group: heads per kv head, or (packed) slabs of 8 heads
    int narrow;                  // d = 128 on the 16x16x32 kernel
};
PrefillPlan prefill_plan(int32_t Hq, int32_t Hkv, int64_t Sq, int32_t d) {
    const int narrow = d == 128 && Sq <= 16;
    const bool k16 = d == 256 || narrow;  // the 16x16x32 kernel
    const int64_t rows = k16 ? 16 : 32, nw = k16 ? kPrefill16Waves : kPrefillWaves;
    const int64_t qt = rows * nw;
    const int group = Hq / Hkv, slabs = (int)((group + nw - 1) / nw);
    const int64_t n_tiles = (Sq + qt - 1) / qt, n_blocks = (Sq + rows - 1) / rows;
    if (narrow || n_blocks * rows * slabs * nw * Hkv < n_tiles * qt * Hq) return {1, (int)n_blocks, slabs, narrow};
    return {0, (int)n_tiles, group, 0};
}

// Key-range splits of a chunked prefill (bf16).  A small chunk has few query
// tiles, so few workgroups walk the whole cache; splitting each tile's key
// range brings the grid to about two rounds of resident workgroups (the
// prefill kernels run one workgroup per CU), keeping at least two key tiles
// per split.  The splits' partials are merged by a combine kernel.
constexpr int kMaxKSplit = 64;
int chunk_ksplit(int32_t B, int32_t Hq, int32_t Hkv, int64_t Sq, int64_t Sk, int32_t d, atf_dtype dtype) {
    if (dtype != ATF_BF16) return 1;
    const PrefillPlan pl = prefill_plan(Hq, Hkv, Sq, d);
    const int64_t active = (int64_t)pl.n_qtiles * B * Hkv * pl.group;  // workgroups with work
    const int64_t kt = (d == 256 || pl.narrow) ? kPrefill16Keys : kPrefillKeys;
    const int64_t cap = std::min<int64_t>(std::max<int64_t>(1, Sk / kt / 2), kMaxKSplit);
    if (active <= 256) return (int)std::max<int64_t>(1, std::min<int64_t>(512 / active, cap));
    // More than one round of resident workgroups (one per CU), the last maybe
    // part-full.  When every query tile walks about the same key range (a
    // chunk after a prefix of at least three times its length), split so the
    // rounds come out fuller: the split count with the fewest rounds per unit
    // of work, kept only if it saves at least 5% (the partials' traffic).
    if (Sk < 4 * Sq) return 1;
    constexpr int64_t kResident = 256;
    auto rounds_per_work = [&](int64_t ns) {
        return (double)((active * ns + kResident - 1) / kResident) / (double)ns;
    };
    int64_t best = 1;
    for (int64_t ns = 2; ns <= std::min<int64_t>(cap, 8); ++ns)
        if (rounds_per_work(ns) < 0.95 * rounds_per_work(best)) best = ns;
    return (int)best;
}

// Prefill key cache (bf16): rotated keys, then transposed values, both laid
// out for S_cap keys per (b, kv head), as in the prepared workspace.
size_t pcache_bytes(int32_t B, int32_t Hkv, int64_t S_cap, int32_t d) {
    return 2 * (size_t)B * Hkv * (size_t)padded_keys(S_cap) * d * 2;
}

// Bytes after the counter (and the prepared keys) that a key-split chunk
// uses: the splits' partials, then (16x16x32 kernel: d = 256, or d = 128
// with at most 16 queries) the queries rotated once for all splits, at a
// 256-byte boundary.
size_t split_partials_bytes(int32_t B, int32_t Hq, int64_t Sq, int32_t d, int ns) {
    return (size_t)B * Hq * (size_t)Sq * ns * (size_t)(d + 2) * sizeof(float);
}
bool split_rotates_queries(int64_t Sq, int32_t d, int ns) { return ns > 1 && (d == 256 || (d == 128 && Sq <= 16)); }
size_t split_extra_bytes(int32_t B, int32_t Hq, int64_t Sq, int32_t d, int ns) {
    if (ns <= 1) return 0;
    size_t n = split_partials_bytes(B, Hq, Sq, d, ns);
    if (split_rotates_queries(Sq, d, ns)) n = (n + 255) / 256 * 256 + (size_t)B * Hq * (size_t)Sq * (d / 2) * 4;
    return n;
}

size_t chunk_ws_bytes(int32_t B, int32_t Hq, int32_t Hkv, int64_t Sq, int64_t Sk, int32_t d, atf_dtype dtype) {
    const int ns = chunk_ksplit(B, Hq, Hkv, Sq, Sk, d, dtype);
    return prefill_ws_bytes(B, Hkv, Sk, d, dtype) + split_extra_bytes(B, Hq, Sq, d, ns);
}

// ---------------------------------------------------------------- decode plan

struct DecodePlan {
    int nsplit = 1;
    int n_slabs = 1;
    int starts[kMaxSplits + 1];
};

// Decode workgroups resident at once: 2 per CU x 256 CUs (every head dim:
// at d = 256 the kernels take 16-key chunks so that two fit).
int64_t decode_resident(int32_t) { return 512; }

int decode_nsplit(int32_t B, int32_t Hq, int32_t Hkv, int64_t S, int32_t d) {
    const int group = Hq / Hkv;
    const int n_slabs = (group + kDecodeHeads - 1) / kDecodeHeads;
    const int64_t units = (int64_t)B * Hkv * n_slabs;
    const int64_t nchunks = (S + kKeyTile - 1) / kKeyTile;
    // aim for one round of resident workgroups; byte-balanced splits then
    // finish together.  Rounded down: one workgroup over the resident count
    // would run as a second round and double the time.  At least one chunk
    // per split.
    int64_t ns = decode_resident(d) / units;
    ns = std::min<int64_t>(ns, kMaxSplits);
    ns = std::min<int64_t>(ns, nchunks);
    return (int)std::max<int64_t>(ns, 1);
}

// Decode workspace: header (counter), the rotated queries ([B*Hq][d/2] bf16
// pair words, rounded up to 256 bytes), then the split partials.
size_t dec_qrot_bytes(int32_t B, int32_t Hq, int32_t d) { return ((size_t)B * Hq * d * 2 + 255) / 256 * 256; }

size_t decode_ws_bytes(int32_t B, int32_t Hq, int32_t Hkv, int64_t S, int32_t d) {
    const int ns = decode_nsplit(B, Hq, Hkv, S, d);
    return kHeaderBytes + dec_qrot_bytes(B, Hq, d) + (size_t)B * Hq * ns * (size_t)(d + 2) * sizeof(float);
}

// Paged, ragged decode: the batch shares a budget of ~512 workgroups per call
// (one round of resident workgroups) in proportion to the sequences' lengths;
// one sequence may take all of it.  The grid is that per-sequence maximum wide.
void paged_plan(int32_t Hq, int32_t Hkv, int64_t max_len, int32_t d, int &budget, int &nsplit_max) {
    const int group = Hq / Hkv;
    const int n_slabs = (group + kDecodeHeads - 1) / kDecodeHeads;
    const int64_t units = (int64_t)Hkv * n_slabs;
    const int64_t nchunks = (max_len + kKeyTile - 1) / kKeyTile;
    const int64_t b = std::max<int64_t>(1, decode_resident(d) / units);  // rounded down, as above
    budget = (int)b;
    nsplit_max = (int)std::max<int64_t>(1, std::min<int64_t>(std::min<int64_t>(b, kMaxSplits), nchunks));
}

size_t paged_ws_bytes(int32_t B, int32_t Hq, int32_t Hkv, int64_t max_len, int32_t d) {
    int budget, ns;
    paged_plan(Hq, Hkv, max_len, d, budget, ns);
    return kHeaderBytes + dec_qrot_bytes(B, Hq, d) + (size_t)B * Hq * ns * (size_t)(d + 2) * sizeof(float);
}

// Algorithmic bytes of keys [0, j) for a query at distance S - j' from key j':
// each key costs 2d bytes of value plus 4 bytes per kept pair.  Pair p (finite
// W_p) is dropped for keys with S - j' > W_p, i.e. j' < S - W_p, so the dropped
// pair-keys below j are sum_p min(j, max(0, S - W_p)).  O(P) per evaluation.
double decode_prefix_bytes(int64_t j, int64_t S, int P, int d, const int *Wi) {
    double dropped = 0.0;
    for (int p = 0; p < P - 1; ++p) {
        const int64_t lim = S - (int64_t)Wi[p];
        if (lim > 0) dropped += (double)std::min(j, lim);
    }
    return (double)j * (2.0 * d + 4.0 * P) - 4.0 * dropped;
}

// Splits of equal ALGORITHMIC bytes: far keys (fewer kept pairs) are cheaper,
// so far splits hold more keys.  Boundaries fall on 64-key chunks and are found
// by binary search on the closed-form prefix, so planning costs
// O(nsplit * P * log(S)) host work however long the cache is.
void plan_decode(int32_t B, int32_t Hq, int32_t Hkv, int64_t S, int32_t d, const int *Wi,
                 DecodePlan &plan) {
    const int P = d / 2;
    const int group = Hq / Hkv;
    plan.n_slabs = (group + kDecodeHeads - 1) / kDecodeHeads;
    plan.nsplit = decode_nsplit(B, Hq, Hkv, S, d);
    const int64_t nchunks = (S + kKeyTile - 1) / kKeyTile;
    auto cum = [&](int64_t c) { return decode_prefix_bytes(std::min(S, c * kKeyTile), S, P, d, Wi); };
    const double total = cum(nchunks);
    plan.starts[0] = 0;
    for (int s = 1; s < plan.nsplit; ++s) {
        const double target = total * s / plan.nsplit;
        // smallest chunk index c with cum(c) >= target (cum is increasing)
        int64_t lo = 0, hi = nchunks;
        while (lo < hi) {
            const int64_t mid = lo + (hi - lo) / 2;
            if (cum(mid) < target) lo = mid + 1; else hi = mid;
        }
        // keep every split non-empty
        const int64_t first = plan.starts[s - 1] / kKeyTile + 1;
        const int64_t last = nchunks - (plan.nsplit - s);
        const int64_t cc = std::max(first, std::min(lo, last));
        plan.starts[s] = (int)(cc * kKeyTile);
    }
    plan.starts[plan.nsplit] = (int)(nchunks * kKeyTile);
}

atf_status hip_status(hipError_t e) { return e == hipSuccess ? ATF_OK : ATF_ERR_HIP; }

atf_status read_counter(unsigned long long *dev, uint64_t *host, hipStream_t s) {
    if (!host) return ATF_OK;
    unsigned long long v = 0;
    if (hipMemcpyAsync(&v, dev, sizeof(v), hipMemcpyDeviceToHost, s) != hipSuccess) return ATF_ERR_HIP;
    if (hipStreamSynchronize(s) != hipSuccess) return ATF_ERR_HIP;
    *host = (uint64_t)v;
    return ATF_OK;
}

// Where a bf16 attention call finds its prepared keys and values.
struct KvView {
    const void *krot, *vt;
    int64_t S_pad;  // keys per (b, kv head) in krot and vt
};

// Attention over prepared keys: Sq query rows that sit at key indices
// Sk - Sq .. Sk - 1 (positions pos0 + Sk - Sq + i), Sk keys at positions
// pos0 + j.  fp32 reads raw k and v; bf16 reads `kv`.  The count goes to
// `counter` (cleared here); a key-range split (n_ksplit > 1) writes its
// partials to `part`.  Shapes and buffers are checked by the caller.
atf_status attend_core(const void *q, const void *k, const void *v, void *out, int32_t B, int32_t Hq,
                       int32_t Hkv, int64_t Sq, int64_t Sk, int32_t d, int32_t layout, double rope_base, double alpha,
                       int32_t causal, int64_t pos0, atf_dtype dtype, const KvView &kv,
                       unsigned long long *counter, float *part, int n_ksplit, uint64_t *skipped_out,
                       hipStream_t s) {
    AttnArgs a;
    std::memset(&a, 0, sizeof(a));
    a.q = q;
    a.out = out;
    a.counter = counter;
    a.B = B;
    a.Hq = Hq;
    a.Hkv = Hkv;
    a.group = Hq / Hkv;
    a.Sq = (int)Sq;
    a.Sk = (int)Sk;
    a.q_pos0 = pos0 + (Sk - Sq);
    a.k_pos0 = pos0;
    a.causal = causal;
    a.gptj = layout;
    a.scale_log2 = (float)(1.4426950408889634 / std::sqrt((double)d));
    window_table_i32(d, rope_base, alpha, a.W);
    theta_table(d, rope_base, a.theta);
    // the count is per call: clear it (the prepared keys may be reused); a
    // key-split short chunk clears it in the query-rotation pass instead
    const bool qrot = dtype == ATF_BF16 && split_rotates_queries(Sq, d, n_ksplit);
    hipError_t e = qrot ? hipSuccess : launch_fill_zero_u64(a.counter, s);
    if (e != hipSuccess) return ATF_ERR_HIP;
    if (dtype == ATF_F32) {
        // the fp32 kernel rotates raw keys itself: `krot` carries k, `vt` carries v
        a.krot = k;
        a.vt = v;
        a.Sk_pad = (int)Sk;
        e = launch_attend_f32(a, d, s);
    } else {
        a.krot = kv.krot;
        a.vt = kv.vt;
        a.Sk_pad = (int)kv.S_pad;
        const PrefillPlan pl = prefill_plan(Hq, Hkv, Sq, d);
        a.hpack = pl.hpack;
        a.narrow = pl.narrow;
        a.n_qtiles = pl.n_qtiles;
        a.group = pl.group;
        a.n_groups = a.n_qtiles * B * Hkv;
        a.n_ksplit = n_ksplit;
        a.part = n_ksplit > 1 ? part : nullptr;
        if (qrot) {
            const size_t off = (split_partials_bytes(B, Hq, Sq, d, n_ksplit) + 255) / 256 * 256;
            a.qrot = (unsigned *)((char *)part + off);
            e = launch_prefill_qrot(a, d, s);
            if (e != hipSuccess) return ATF_ERR_HIP;
        }
        e = launch_prefill_bf16(a, d, s);
    }
    if (e != hipSuccess) return ATF_ERR_HIP;
    return read_counter(a.counter, skipped_out, s);
}

// attend_core over the workspace of atf_prefill_prepare_kv: counter in the
// header, then K' and V^T for Sk keys, then (split) the partials.
atf_status attend_impl(const void *q, const void *k, const void *v, void *out, int32_t B, int32_t Hq,
                       int32_t Hkv, int64_t Sq, int64_t Sk, int32_t d, int32_t layout, double rope_base, double alpha,
                       int32_t causal, int64_t pos0, atf_dtype dtype, void *workspace, size_t workspace_bytes,
                       uint64_t *skipped_out, hipStream_t s, int n_ksplit = 1) {
    if (!aligned16(q) || !aligned16(out)) return ATF_ERR_INVALID_ARG;
    if (dtype == ATF_F32 && (!aligned16(k) || !aligned16(v))) return ATF_ERR_INVALID_ARG;
    if (!aligned16(workspace) || workspace_bytes < prefill_ws_bytes(B, Hkv, Sk, d, dtype))
        return ATF_ERR_WORKSPACE;
    char *ws = (char *)workspace + kHeaderBytes;
    const int64_t S_pad = padded_keys(Sk);
    const KvView kv{ws, ws + (size_t)B * Hkv * (size_t)S_pad * d * 2, S_pad};
    float *part = (float *)((char *)workspace + prefill_ws_bytes(B, Hkv, Sk, d, dtype));
    return attend_core(q, k, v, out, B, Hq, Hkv, Sq, Sk, d, layout, rope_base, alpha, causal, pos0, dtype, kv,
                       (unsigned long long *)workspace, part, n_ksplit, skipped_out, s);
}

// Checks shared by the paged decode entry points (everything but the scratch).
atf_status paged_decode_checks(const void *q, const void *kpool, const void *vpool, const void *out,
                               const int32_t *page_table, const int32_t *seq_lens, int32_t max_pages,
                               int32_t num_pages, int32_t B, int32_t Hq, int32_t Hkv, int64_t max_len, int32_t d,
                               int32_t rope_layout, double rope_base, double alpha, int32_t causal, int64_t pos0,
                               atf_dtype dtype) {
    atf_status st = check_shape(B, Hq, Hkv, max_len, d, rope_base, alpha, causal, pos0, dtype);
    if (st != ATF_OK) return st;
    if (bad_layout(rope_layout)) return ATF_ERR_INVALID_ARG;
    if (!page_table || !seq_lens || ((uintptr_t)page_table & 3u) != 0 || ((uintptr_t)seq_lens & 3u) != 0)
        return ATF_ERR_INVALID_ARG;
    if (max_pages < 1 || num_pages < 1 || max_len > (int64_t)max_pages * kKeyTile) return ATF_ERR_INVALID_ARG;
    if (!aligned16(q) || !aligned16(kpool) || !aligned16(vpool) || !aligned16(out)) return ATF_ERR_INVALID_ARG;
    if (dtype != ATF_BF16) return ATF_ERR_UNSUPPORTED;
    return ATF_OK;
}

// Paged decode over a checked shape with `workspace` (at least paged_ws_bytes):
// counter, rotated queries, split partials.
atf_status paged_decode_launch(const void *q, const void *kpool, const void *vpool, void *out,
                               const int32_t *page_table, const int32_t *seq_lens, int32_t max_pages,
                               int32_t num_pages, int32_t B, int32_t Hq, int32_t Hkv, int64_t max_len, int32_t d,
                               int32_t rope_layout, double rope_base, double alpha, int64_t pos0, void *workspace,
                               uint64_t *skipped_out, hipStream_t s) {
    DecodeArgs a;
    std::memset(&a, 0, sizeof(a));
    a.q = q;
    a.k = kpool;
    a.v = vpool;
    a.out = out;
    a.counter = (unsigned long long *)workspace;
    a.qrot = (unsigned *)((char *)workspace + kHeaderBytes);
    a.part = (float *)((char *)workspace + kHeaderBytes + dec_qrot_bytes(B, Hq, d));
    a.B = B;
    a.Hq = Hq;
    a.Hkv = Hkv;
    a.group = Hq / Hkv;
    a.S = (int)max_len;
    a.page_table = page_table;
    a.seq_lens = seq_lens;
    a.max_pages = max_pages;
    a.num_pages = num_pages;
    a.pos0 = pos0;
    a.gptj = rope_layout;
    a.scale_log2 = (float)(1.4426950408889634 / std::sqrt((double)d));
    window_table_i32(d, rope_base, alpha, a.W);
    theta_table(d, rope_base, a.theta);
    a.n_slabs = (a.group + kDecodeHeads - 1) / kDecodeHeads;
    paged_plan(Hq, Hkv, max_len, d, a.split_budget, a.nsplit);
    if (launch_decode_paged_bf16(a, d, s) != hipSuccess) return ATF_ERR_HIP;
    return read_counter(a.counter, skipped_out, s);
}

}  // namespace

extern "C" {

const char *atf_status_string(atf_status s) {
    switch (s) {
        case ATF_OK: return "ATF_OK";
        case ATF_ERR_INVALID_ARG: return "ATF_ERR_INVALID_ARG";
        case ATF_ERR_UNSUPPORTED: return "ATF_ERR_UNSUPPORTED";
        case ATF_ERR_WORKSPACE: return "ATF_ERR_WORKSPACE";
        case ATF_ERR_HIP: return "ATF_ERR_HIP";
    }
    return "ATF_UNKNOWN_STATUS";
}

const char *atf_version(void) { return "rfw-atf 0.1 gfx950"; }

atf_status atf_window_table(int32_t d, double rope_base, double alpha, int64_t *W_out) {
    if (!W_out || d < 2 || (d & 1) || d > 65536) return ATF_ERR_INVALID_ARG;
    if (!std::isfinite(rope_base) || !(rope_base > 1.0)) return ATF_ERR_INVALID_ARG;
    if (std::isnan(alpha) || !(alpha > 0.0)) return ATF_ERR_INVALID_ARG;
    window_table(d, rope_base, alpha, W_out);
    return ATF_OK;
}

atf_status atf_skipped_pair_products(int64_t S, int32_t d, double rope_base, double alpha,
                                     int32_t causal, int32_t is_decode, uint64_t *per_head_out) {
    if (!per_head_out || S < 1 || (is_decode != 0 && is_decode != 1)) return ATF_ERR_INVALID_ARG;
    if (causal != 0 && causal != 1) return ATF_ERR_INVALID_ARG;
    std::vector<int64_t> W((size_t)std::max(1, d / 2));
    atf_status st = atf_window_table(d, rope_base, alpha, W.data());
    if (st != ATF_OK) return st;
    uint64_t total = 0;
    for (int64_t w : W) {
        if (w == kInf64) continue;
        // distances 1..S-1 occur S - t times in prefill; decode sees 1..S once each
        const int64_t n = is_decode ? S - w : S - 1 - w;
        if (n <= 0) continue;
        total += is_decode ? (uint64_t)n : (uint64_t)n * (uint64_t)(n + 1) / 2u;
    }
    // without the causal mask a prefill query also sees the keys after it, at
    // the same distances: twice the count (decode has no key after its query)
    if (causal == 0 && !is_decode) total *= 2u;
    *per_head_out = total;
    return ATF_OK;
}

size_t atf_prefill_workspace_bytes(int32_t B, int32_t Hkv, int64_t S, int32_t d, atf_dtype dtype) {
    if (B < 1 || Hkv < 1 || S < 1 || (!supported_d(d))) return 0;
    if (dtype != ATF_F32 && dtype != ATF_BF16) return 0;
    return prefill_ws_bytes(B, Hkv, S, d, dtype);
}

atf_status atf_prefill_prepare_kv(const void *k, const void *v, int32_t B, int32_t Hkv, int64_t S,
                                  int32_t d, int32_t rope_layout, double rope_base, int64_t pos0, atf_dtype dtype,
                                  void *workspace, size_t workspace_bytes, atf_stream_t stream) {
    atf_status st = check_shape(B, Hkv, Hkv, S, d, rope_base, 1.0, 1, pos0, dtype);
    if (st != ATF_OK) return st;
    if (bad_layout(rope_layout)) return ATF_ERR_INVALID_ARG;
    if (!aligned16(k) || !aligned16(v)) return ATF_ERR_INVALID_ARG;
    if (!aligned16(workspace) || workspace_bytes < prefill_ws_bytes(B, Hkv, S, d, dtype))
        return ATF_ERR_WORKSPACE;
    PrepArgs a;
    std::memset(&a, 0, sizeof(a));
    a.k = k;
    a.v = v;
    a.counter = (unsigned long long *)workspace;
    a.B = B;
    a.Hkv = Hkv;
    a.S = (int)S;
    a.S_pad = (int)padded_keys(S);
    a.k_begin = 0;
    a.k_end = a.src_rows = (int)S;
    a.tile0 = 0;
    a.n_tiles = a.S_pad / kKeyTile;
    a.pos0 = pos0;
    a.gptj = rope_layout;
    theta_table(d, rope_base, a.theta);
    hipStream_t s = (hipStream_t)stream;
    if (dtype == ATF_F32) return hip_status(launch_prep_f32(a, d, s));
    char *ws = (char *)workspace + kHeaderBytes;
    const size_t per = (size_t)B * Hkv * (size_t)a.S_pad * d * 2;
    a.krot = ws;
    a.vt = ws + per;
    return hip_status(launch_prep_bf16(a, d, s));
}

atf_status atf_prefill_attend(const void *q, const void *k, const void *v, void *out, int32_t B, int32_t Hq,
                              int32_t Hkv, int64_t S, int32_t d, int32_t rope_layout, double rope_base, double alpha,
                              int32_t causal, int64_t pos0, atf_dtype dtype, void *workspace,
                              size_t workspace_bytes, uint64_t *skipped_out, atf_stream_t stream) {
    atf_status st = check_shape(B, Hq, Hkv, S, d, rope_base, alpha, causal, pos0, dtype);
    if (st != ATF_OK) return st;
    if (bad_layout(rope_layout)) return ATF_ERR_INVALID_ARG;
    return attend_impl(q, k, v, out, B, Hq, Hkv, S, S, d, rope_layout, rope_base, alpha, causal, pos0, dtype, workspace,
                       workspace_bytes, skipped_out, stream);
}

atf_status atf_prefill(const void *q, const void *k, const void *v, void *out, int32_t B,
                       int32_t Hq, int32_t Hkv, int64_t S, int32_t d, int32_t rope_layout, double rope_base,
                       double alpha, int32_t causal, int64_t pos0, atf_dtype dtype,
                       void *workspace, size_t workspace_bytes, uint64_t *skipped_out,
                       atf_stream_t stream) {
    atf_status st = check_shape(B, Hq, Hkv, S, d, rope_base, alpha, causal, pos0, dtype);
    if (st != ATF_OK) return st;
    if (bad_layout(rope_layout)) return ATF_ERR_INVALID_ARG;
    if (!aligned16(q) || !aligned16(k) || !aligned16(v) || !aligned16(out)) return ATF_ERR_INVALID_ARG;
    if (!aligned16(workspace) || workspace_bytes < prefill_ws_bytes(B, Hkv, S, d, dtype))
        return ATF_ERR_WORKSPACE;
    st = atf_prefill_prepare_kv(k, v, B, Hkv, S, d, rope_layout, rope_base, pos0, dtype, workspace,
                                workspace_bytes, stream);
    if (st != ATF_OK) return st;
    return atf_prefill_attend(q, k, v, out, B, Hq, Hkv, S, d, rope_layout, rope_base, alpha, causal, pos0, dtype,
                              workspace, workspace_bytes, skipped_out, stream);
}

atf_status atf_prefill_chunk(const void *q, const void *k, const void *v, void *out, int32_t B,
                             int32_t Hq, int32_t Hkv, int64_t Sq, int64_t Sk, int32_t d, int32_t rope_layout,
                             double rope_base, double alpha, int32_t causal, int64_t pos0, atf_dtype dtype,
                             void *workspace, size_t workspace_bytes, uint64_t *skipped_out, atf_stream_t stream) {
    if (Sq < 1 || Sq > Sk) return ATF_ERR_INVALID_ARG;
    atf_status st = check_shape(B, Hq, Hkv, Sk, d, rope_base, alpha, causal, pos0, dtype);
    if (st != ATF_OK) return st;
    if (bad_layout(rope_layout)) return ATF_ERR_INVALID_ARG;
    if (!aligned16(q) || !aligned16(k) || !aligned16(v) || !aligned16(out)) return ATF_ERR_INVALID_ARG;
    if (!aligned16(workspace) || workspace_bytes < prefill_ws_bytes(B, Hkv, Sk, d, dtype))
        return ATF_ERR_WORKSPACE;
    st = atf_prefill_prepare_kv(k, v, B, Hkv, Sk, d, rope_layout, rope_base, pos0, dtype, workspace,
                                workspace_bytes, stream);
    if (st != ATF_OK) return st;
    // split the key range when the workspace has room for the partials
    const int ns = workspace_bytes >= chunk_ws_bytes(B, Hq, Hkv, Sq, Sk, d, dtype)
                       ? chunk_ksplit(B, Hq, Hkv, Sq, Sk, d, dtype) : 1;
    return attend_impl(q, k, v, out, B, Hq, Hkv, Sq, Sk, d, rope_layout, rope_base, alpha, causal, pos0, dtype,
                       workspace, workspace_bytes, skipped_out, (hipStream_t)stream, ns);
}

size_t atf_prefill_chunk_workspace_bytes(int32_t B, int32_t Hq, int32_t Hkv, int64_t Sq, int64_t Sk, int32_t d,
                                         atf_dtype dtype) {
    if (B < 1 || Hq < 1 || Hkv < 1 || Hq % Hkv != 0 || Sq < 1 || Sq > Sk || (!supported_d(d))) return 0;
    if (dtype != ATF_F32 && dtype != ATF_BF16) return 0;
    return chunk_ws_bytes(B, Hq, Hkv, Sq, Sk, d, dtype);
}

size_t atf_prefill_cache_bytes(int32_t B, int32_t Hkv, int64_t S_cap, int32_t d) {
    if (B < 1 || Hkv < 1 || S_cap < 1 || padded_keys(S_cap) >= (int64_t)INT32_MAX || (!supported_d(d))) return 0;
    return pcache_bytes(B, Hkv, S_cap, d);
}

atf_status atf_prefill_cache_append(const void *k, const void *v, int32_t B, int32_t Hkv, int64_t n, int64_t k_begin,
                                    int64_t S_cap, int32_t d, int32_t rope_layout, double rope_base, int64_t pos0,
                                    void *cache, size_t cache_bytes, atf_stream_t stream) {
    if (n < 1 || k_begin < 0 || k_begin > S_cap - n) return ATF_ERR_INVALID_ARG;
    atf_status st = check_shape(B, Hkv, Hkv, S_cap, d, rope_base, 1.0, 1, pos0, ATF_BF16);
    if (st != ATF_OK) return st;
    if (bad_layout(rope_layout)) return ATF_ERR_INVALID_ARG;
    if (!aligned16(k) || !aligned16(v)) return ATF_ERR_INVALID_ARG;
    if (!aligned16(cache) || cache_bytes < pcache_bytes(B, Hkv, S_cap, d)) return ATF_ERR_WORKSPACE;
    PrepArgs a;
    std::memset(&a, 0, sizeof(a));
    a.k = k;
    a.v = v;
    a.B = B;
    a.Hkv = Hkv;
    a.S = (int)S_cap;
    a.S_pad = (int)padded_keys(S_cap);
    a.k_begin = (int)k_begin;
    a.k_end = (int)(k_begin + n);
    a.src_rows = (int)n;
    // from the tile holding k_begin to the end of the attention tile holding
    // the last key: the keys after it in that tile are cleared
    a.tile0 = (int)(k_begin / kKeyTile);
    a.n_tiles = (int)(std::min<int64_t>(a.S_pad, padded_keys(k_begin + n)) / kKeyTile) - a.tile0;
    a.pos0 = pos0;
    a.gptj = rope_layout;
    theta_table(d, rope_base, a.theta);
    char *c = (char *)cache;
    a.krot = c;
    a.vt = c + pcache_bytes(B, Hkv, S_cap, d) / 2;
    return hip_status(launch_prep_bf16(a, d, (hipStream_t)stream));
}

size_t atf_prefill_cached_scratch_bytes(int32_t B, int32_t Hq, int32_t Hkv, int64_t Sq, int64_t Sk, int32_t d) {
    if (B < 1 || Hq < 1 || Hkv < 1 || Hq % Hkv != 0 || Sq < 1 || Sq > Sk || (!supported_d(d))) return 0;
    const int ns = chunk_ksplit(B, Hq, Hkv, Sq, Sk, d, ATF_BF16);
    return kHeaderBytes + split_extra_bytes(B, Hq, Sq, d, ns);
}

atf_status atf_prefill_chunk_cached(const void *q, void *out, int32_t B, int32_t Hq, int32_t Hkv, int64_t Sq,
                                    int64_t Sk, int64_t S_cap, int32_t d, int32_t rope_layout, double rope_base,
                                    double alpha, int32_t causal, int64_t pos0, const void *cache,
                                    size_t cache_bytes, void *scratch, size_t scratch_bytes, uint64_t *skipped_out,
                                    atf_stream_t stream) {
    if (Sq < 1 || Sq > Sk || Sk > S_cap) return ATF_ERR_INVALID_ARG;
    atf_status st = check_shape(B, Hq, Hkv, S_cap, d, rope_base, alpha, causal, pos0, ATF_BF16);
    if (st != ATF_OK) return st;
    if (bad_layout(rope_layout)) return ATF_ERR_INVALID_ARG;
    if (!aligned16(q) || !aligned16(out)) return ATF_ERR_INVALID_ARG;
    if (!aligned16(cache) || cache_bytes < pcache_bytes(B, Hkv, S_cap, d)) return ATF_ERR_WORKSPACE;
    if (!aligned16(scratch) || scratch_bytes < kHeaderBytes) return ATF_ERR_WORKSPACE;
    // split the key range when the scratch has room for the partials
    const int ns = scratch_bytes >= atf_prefill_cached_scratch_bytes(B, Hq, Hkv, Sq, Sk, d)
                       ? chunk_ksplit(B, Hq, Hkv, Sq, Sk, d, ATF_BF16) : 1;
    const int64_t S_pad = padded_keys(S_cap);
    const char *c = (const char *)cache;
    const KvView kv{c, c + pcache_bytes(B, Hkv, S_cap, d) / 2, S_pad};
    return attend_core(q, nullptr, nullptr, out, B, Hq, Hkv, Sq, Sk, d, rope_layout, rope_base, alpha, causal, pos0,
                       ATF_BF16, kv, (unsigned long long *)scratch, (float *)((char *)scratch + kHeaderBytes), ns,
                       skipped_out, (hipStream_t)stream);
}

size_t atf_decode_workspace_bytes(int32_t B, int32_t Hq, int32_t Hkv, int64_t S, int32_t d) {
    if (B < 1 || Hq < 1 || Hkv < 1 || Hq % Hkv != 0 || S < 1 || (!supported_d(d))) return 0;
    return decode_ws_bytes(B, Hq, Hkv, S, d);
}

atf_status atf_decode(const void *q, const void *k, const void *v, void *out, int32_t B,
                      int32_t Hq, int32_t Hkv, int64_t S, int32_t d, int32_t rope_layout, double rope_base,
                      double alpha, int32_t causal, int64_t pos0, atf_dtype dtype, void *workspace,
                      size_t workspace_bytes, uint64_t *skipped_out, atf_stream_t stream) {
    atf_status st = check_shape(B, Hq, Hkv, S, d, rope_base, alpha, causal, pos0, dtype);
    if (st != ATF_OK) return st;
    if (bad_layout(rope_layout)) return ATF_ERR_INVALID_ARG;
    if (!aligned16(q) || !aligned16(k) || !aligned16(v) || !aligned16(out)) return ATF_ERR_INVALID_ARG;
    if (!aligned16(workspace) || workspace_bytes < decode_ws_bytes(B, Hq, Hkv, S, d))
        return ATF_ERR_WORKSPACE;
    hipStream_t s = (hipStream_t)stream;
    unsigned long long *counter = (unsigned long long *)workspace;
    if (dtype == ATF_F32) {
        AttnArgs a;
        std::memset(&a, 0, sizeof(a));
        a.q = q;
        a.krot = k;
        a.vt = v;
        a.out = out;
        a.counter = counter;
        a.B = B;
        a.Hq = Hq;
        a.Hkv = Hkv;
        a.group = Hq / Hkv;
        a.Sq = 1;
        a.Sk = (int)S;
        a.Sk_pad = (int)S;
        a.q_pos0 = pos0 + S;
        a.k_pos0 = pos0;
        a.causal = 1;  // the query follows every key: both settings see all of them
        a.gptj = rope_layout;
        a.scale_log2 = (float)(1.4426950408889634 / std::sqrt((double)d));
        window_table_i32(d, rope_base, alpha, a.W);
        theta_table(d, rope_base, a.theta);
        if (launch_fill_zero_u64(counter, s) != hipSuccess) return ATF_ERR_HIP;
        if (launch_attend_f32(a, d, s) != hipSuccess) return ATF_ERR_HIP;
        return read_counter(counter, skipped_out, s);
    }
    DecodeArgs a;
    std::memset(&a, 0, sizeof(a));
    a.q = q;
    a.k = k;
    a.v = v;
    a.out = out;
    a.counter = counter;
    a.qrot = (unsigned *)((char *)workspace + kHeaderBytes);
    a.part = (float *)((char *)workspace + kHeaderBytes + dec_qrot_bytes(B, Hq, d));
    a.B = B;
    a.Hq = Hq;
    a.Hkv = Hkv;
    a.group = Hq / Hkv;
    a.S = (int)S;
    a.pos0 = pos0;
    a.gptj = rope_layout;
    a.scale_log2 = (float)(1.4426950408889634 / std::sqrt((double)d));
    window_table_i32(d, rope_base, alpha, a.W);
    theta_table(d, rope_base, a.theta);
    DecodePlan plan;
    plan_decode(B, Hq, Hkv, S, d, a.W, plan);
    a.nsplit = plan.nsplit;
    a.n_slabs = plan.n_slabs;
    std::memcpy(a.split_start, plan.starts, sizeof(int) * (size_t)(plan.nsplit + 1));
    if (launch_decode_bf16(a, d, s) != hipSuccess) return ATF_ERR_HIP;
    return read_counter(counter, skipped_out, s);
}

size_t atf_decode_kcache_bytes(int32_t B, int32_t Hkv, int64_t cap, int32_t d) {
    if (B < 1 || Hkv < 1 || cap < kKeyTile || cap % kKeyTile != 0 || cap >= (int64_t)INT32_MAX) return 0;
    if (!supported_d(d)) return 0;
    return (size_t)B * Hkv * (size_t)cap * d * 2;
}

atf_status atf_decode_pack_k(const void *k, void *kcache, int32_t B, int32_t Hkv, int64_t n, int64_t k_begin,
                             int64_t cap, int32_t d, int32_t rope_layout, double rope_base, int64_t pos0,
                             atf_dtype dtype, atf_stream_t stream) {
    return atf_decode_append_kv(k, nullptr, kcache, nullptr, B, Hkv, n, k_begin, cap, d, rope_layout, rope_base, pos0,
                                dtype, stream);
}

atf_status atf_decode_append_kv(const void *k, const void *v, void *kcache, void *vcache, int32_t B, int32_t Hkv,
                                int64_t n, int64_t k_begin, int64_t cap, int32_t d, int32_t rope_layout,
                                double rope_base, int64_t pos0, atf_dtype dtype, atf_stream_t stream) {
    if ((v == nullptr) != (vcache == nullptr)) return ATF_ERR_INVALID_ARG;
    if (v && (!aligned16(v) || !aligned16(vcache))) return ATF_ERR_INVALID_ARG;
    if (bad_layout(rope_layout)) return ATF_ERR_INVALID_ARG;
    if (!k || !kcache || !aligned16(k) || !aligned16(kcache)) return ATF_ERR_INVALID_ARG;
    if (B < 1 || Hkv < 1 || n < 1 || k_begin < 0) return ATF_ERR_INVALID_ARG;
    if (cap < kKeyTile || cap % kKeyTile != 0 || k_begin + n > cap) return ATF_ERR_INVALID_ARG;
    if (d < 2 || (d & 1)) return ATF_ERR_INVALID_ARG;
    if (!std::isfinite(rope_base) || !(rope_base > 1.0)) return ATF_ERR_INVALID_ARG;
    if (dtype != ATF_F32 && dtype != ATF_BF16) return ATF_ERR_INVALID_ARG;
    if (pos0 < 0 || pos0 + cap + 1 >= (int64_t)INT32_MAX) return ATF_ERR_INVALID_ARG;
    if (!supported_d(d)) return ATF_ERR_UNSUPPORTED;
    if (dtype != ATF_BF16) return ATF_ERR_UNSUPPORTED;
    KPackArgs a;
    std::memset(&a, 0, sizeof(a));
    a.k = k;
    a.kc = kcache;
    a.v = v;
    a.vc = vcache;
    a.B = B;
    a.Hkv = Hkv;
    a.n = (int)n;
    a.cap = (int)cap;
    a.k_begin = k_begin;
    a.pos0 = pos0;
    a.gptj = rope_layout;
    theta_table(d, rope_base, a.theta);
    return hip_status(launch_kpack_bf16(a, d, (hipStream_t)stream));
}

atf_status atf_decode_kcache(const void *q, const void *kcache, const void *v, void *out, int32_t B,
                             int32_t Hq, int32_t Hkv, int64_t S, int64_t cap, int32_t d, int32_t rope_layout,
                             double rope_base, double alpha, int32_t causal, int64_t pos0, atf_dtype dtype,
                             void *workspace, size_t workspace_bytes, uint64_t *skipped_out, atf_stream_t stream) {
    atf_status st = check_shape(B, Hq, Hkv, S, d, rope_base, alpha, causal, pos0, dtype);
    if (st != ATF_OK) return st;
    if (bad_layout(rope_layout)) return ATF_ERR_INVALID_ARG;
    if (cap < kKeyTile || cap % kKeyTile != 0 || S > cap || pos0 + cap + 1 >= (int64_t)INT32_MAX)
        return ATF_ERR_INVALID_ARG;
    if (!aligned16(q) || !aligned16(kcache) || !aligned16(v) || !aligned16(out)) return ATF_ERR_INVALID_ARG;
    if (dtype != ATF_BF16) return ATF_ERR_UNSUPPORTED;
    if (!aligned16(workspace) || workspace_bytes < decode_ws_bytes(B, Hq, Hkv, S, d)) return ATF_ERR_WORKSPACE;
    hipStream_t s = (hipStream_t)stream;
    DecodeArgs a;
    std::memset(&a, 0, sizeof(a));
    a.q = q;
    a.k = kcache;
    a.v = v;
    a.out = out;
    a.counter = (unsigned long long *)workspace;
    a.qrot = (unsigned *)((char *)workspace + kHeaderBytes);
    a.part = (float *)((char *)workspace + kHeaderBytes + dec_qrot_bytes(B, Hq, d));
    a.B = B;
    a.Hq = Hq;
    a.Hkv = Hkv;
    a.group = Hq / Hkv;
    a.S = (int)S;
    a.cap = (int)cap;
    a.pos0 = pos0;
    a.gptj = rope_layout;
    a.scale_log2 = (float)(1.4426950408889634 / std::sqrt((double)d));
    window_table_i32(d, rope_base, alpha, a.W);
    theta_table(d, rope_base, a.theta);
    DecodePlan plan;
    plan_decode(B, Hq, Hkv, S, d, a.W, plan);
    a.nsplit = plan.nsplit;
    a.n_slabs = plan.n_slabs;
    std::memcpy(a.split_start, plan.starts, sizeof(int) * (size_t)(plan.nsplit + 1));
    if (launch_decode_kcache_bf16(a, d, s) != hipSuccess) return ATF_ERR_HIP;
    return read_counter(a.counter, skipped_out, s);
}

size_t atf_decode_paged_workspace_bytes(int32_t B, int32_t Hq, int32_t Hkv, int64_t max_len, int32_t d) {
    if (check_shape(B, Hq, Hkv, max_len, d, 2.0, 1.0, 1, 0, ATF_BF16) != ATF_OK) return 0;
    return paged_ws_bytes(B, Hq, Hkv, max_len, d);
}

size_t atf_paged_page_bytes(int32_t Hkv, int32_t d) {
    if (Hkv < 1 || (!supported_d(d))) return 0;
    return (size_t)Hkv * kKeyTile * d * 2;
}

atf_status atf_paged_write(const void *k, const void *v, void *kpool, void *vpool, const int32_t *page_table,
                           int32_t max_pages, int32_t num_pages, int32_t B, int32_t Hkv, int64_t n, int64_t k_begin,
                           int32_t d, int32_t rope_layout, double rope_base, int64_t pos0, atf_dtype dtype,
                           atf_stream_t stream) {
    if (!k || !v || !kpool || !vpool || !page_table) return ATF_ERR_INVALID_ARG;
    if (bad_layout(rope_layout)) return ATF_ERR_INVALID_ARG;
    if (!aligned16(k) || !aligned16(v) || !aligned16(kpool) || !aligned16(vpool) ||
        ((uintptr_t)page_table & 3u) != 0)
        return ATF_ERR_INVALID_ARG;
    if (B < 1 || Hkv < 1 || n < 1 || k_begin < 0 || max_pages < 1 || num_pages < 1) return ATF_ERR_INVALID_ARG;
    const int64_t cap = (int64_t)max_pages * kKeyTile;
    if (k_begin + n > cap) return ATF_ERR_INVALID_ARG;
    if (d < 2 || (d & 1)) return ATF_ERR_INVALID_ARG;
    if (!std::isfinite(rope_base) || !(rope_base > 1.0)) return ATF_ERR_INVALID_ARG;
    if (dtype != ATF_F32 && dtype != ATF_BF16) return ATF_ERR_INVALID_ARG;
    if (pos0 < 0 || pos0 + cap + 1 >= (int64_t)INT32_MAX) return ATF_ERR_INVALID_ARG;
    if (!supported_d(d)) return ATF_ERR_UNSUPPORTED;
    if (dtype != ATF_BF16) return ATF_ERR_UNSUPPORTED;
    PagedWriteArgs a;
    std::memset(&a, 0, sizeof(a));
    a.k = k;
    a.v = v;
    a.kpool = kpool;
    a.vpool = vpool;
    a.page_table = page_table;
    a.B = B;
    a.Hkv = Hkv;
    a.n = (int)n;
    a.max_pages = max_pages;
    a.num_pages = num_pages;
    a.k_begin = k_begin;
    a.pos0 = pos0;
    a.gptj = rope_layout;
    theta_table(d, rope_base, a.theta);
    return hip_status(launch_paged_write_bf16(a, d, (hipStream_t)stream));
}

atf_status atf_decode_paged(const void *q, const void *kpool, const void *vpool, void *out,
                            const int32_t *page_table, const int32_t *seq_lens, int32_t max_pages, int32_t num_pages,
                            int32_t B, int32_t Hq, int32_t Hkv, int64_t max_len, int32_t d, int32_t rope_layout,
                            double rope_base, double alpha, int32_t causal, int64_t pos0, atf_dtype dtype,
                            void *workspace, size_t workspace_bytes, uint64_t *skipped_out, atf_stream_t stream) {
    atf_status st = paged_decode_checks(q, kpool, vpool, out, page_table, seq_lens, max_pages, num_pages, B, Hq, Hkv,
                                        max_len, d, rope_layout, rope_base, alpha, causal, pos0, dtype);
    if (st != ATF_OK) return st;
    if (!aligned16(workspace) || workspace_bytes < paged_ws_bytes(B, Hq, Hkv, max_len, d))
        return ATF_ERR_WORKSPACE;
    return paged_decode_launch(q, kpool, vpool, out, page_table, seq_lens, max_pages, num_pages, B, Hq, Hkv,
                               max_len, d, rope_layout, rope_base, alpha, pos0, workspace, skipped_out,
                               (hipStream_t)stream);
}

atf_status atf_decode_paged_noalloc(const void *q, const void *kpool, const void *vpool, void *out,
                                    const int32_t *page_table, const int32_t *seq_lens, int32_t max_pages,
                                    int32_t num_pages, int32_t B, int32_t Hq, int32_t Hkv, int64_t max_len,
                                    int32_t d, int32_t rope_layout, double rope_base, double alpha, int32_t causal,
                                    int64_t pos0, atf_dtype dtype, uint64_t *skipped_out, atf_stream_t stream) {
    atf_status st = paged_decode_checks(q, kpool, vpool, out, page_table, seq_lens, max_pages, num_pages, B, Hq, Hkv,
                                        max_len, d, rope_layout, rope_base, alpha, causal, pos0, dtype);
    if (st != ATF_OK) return st;
    // the shape must fit the library's scratch; checked before any HIP call
    if (paged_ws_bytes(B, Hq, Hkv, max_len, d) > (size_t)ATF_NOALLOC_SCRATCH_BYTES) return ATF_ERR_WORKSPACE;
    hipStream_t s = (hipStream_t)stream;
    void *scratch = nullptr;
    if (noalloc_scratch(s, &scratch) != hipSuccess) return ATF_ERR_HIP;
    if (!scratch) return ATF_ERR_INVALID_ARG;  // the stream belongs to another device than the current one
    return paged_decode_launch(q, kpool, vpool, out, page_table, seq_lens, max_pages, num_pages, B, Hq, Hkv,
                               max_len, d, rope_layout, rope_base, alpha, pos0, scratch, skipped_out, s);
}

}  // extern "C"
