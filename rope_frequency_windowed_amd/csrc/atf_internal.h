// Internal interface between the host planner (atf_api.cpp) and the HIP
// kernels (atf_kernels.hip).  Not part of the public ABI.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace atf {

constexpr int kMaxPairs = 128;    // d <= 256
constexpr int kKeyTile = 64;      // keys per prefill tile / decode chunk
#ifndef ATF_PREFILL_WAVES
#define ATF_PREFILL_WAVES 8
#endif
#ifndef ATF_PREFILL_KEYS
#define ATF_PREFILL_KEYS 128
#endif
// bf16 prefill, d <= 128: MFMA 32x32x16, 32 queries per wave
constexpr int kPrefillWaves = ATF_PREFILL_WAVES;       // waves per workgroup
constexpr int kPrefillKeys = ATF_PREFILL_KEYS;         // keys per LDS tile
// bf16 prefill, d = 256: MFMA 16x16x32, 16 queries per wave.  With 32 queries
// a wave's query fragments and accumulators would need one wave per SIMD; 16
// queries fit two per SIMD.  64-key tiles keep the double buffer at 128 KB.
constexpr int kPrefill16Waves = 8;
constexpr int kPrefill16Keys = 64;
constexpr int kQueryTileF32 = 64; // queries per prefill workgroup (fp32)
constexpr int kMaxSplits = 256;   // decode splits per (batch, kv head)
constexpr int kDecodeHeads = 8;   // query heads one decode workgroup serves
constexpr int kWindowInf = 0x7fffffff;
// Library-owned device scratch of atf_decode_paged_noalloc, per GPU.
constexpr size_t kNoAllocScratchBytes = (size_t)32 << 20;

// Padded key count: every tile is full, padding rows hold zeros.
// rotated-key / transposed-value rows kept per (b, kv head): whole prefill tiles
inline int64_t padded_keys(int64_t S) { return (S + kPrefillKeys - 1) / kPrefillKeys * kPrefillKeys; }

// Arguments of the key/value preparation pass.
struct PrepArgs {
    const void *k;
    const void *v;
    void *krot;                       // rotated keys [B][Hkv][S_pad][d]
    void *vt;                         // bf16 only: transposed value tiles
    unsigned long long *counter;      // zeroed here (nullable)
    int B, Hkv, S, S_pad;             // S: fp32 rows; S_pad: keys per (b, h) in krot / vt
    int k_begin, k_end, src_rows;     // bf16: keys [k_begin, k_end) from src_rows rows per (b, h)
    int tile0, n_tiles;               // bf16: 64-key tiles written: [tile0, tile0 + n_tiles)
    long long pos0;
    int gptj;                         // rotary pairs: 0 = dims (p, p + d/2), 1 = dims (2p, 2p + 1)
    double theta[kMaxPairs];
};

// Arguments of the attention kernels (prefill; the fp32 kernel also decodes).
struct AttnArgs {
    const void *q;
    const void *krot;                 // from the preparation pass
    const void *vt;                   // bf16: transposed value tiles; fp32: v itself
    void *out;
    unsigned long long *counter;      // dropped (query, key, pair) terms
    int B, Hq, Hkv, group;
    int Sq, Sk, Sk_pad;               // query rows, keys, padded keys
    long long q_pos0, k_pos0;         // position of query 0 and key 0
    int causal;                       // 1: keys at or before the query; 0: all keys, windows on |i - j|
    int gptj;                         // rotary pairs: 0 = dims (p, p + d/2), 1 = dims (2p, 2p + 1)
    int n_qtiles, n_groups;           // work decomposition
    int n_ksplit;                     // key-range splits (grid.y); > 1: partials to `part`, then a combine
    int hpack;                        // 1: a work item is one query block of up to 8 heads sharing a kv head
    int narrow;                       // 1: d = 128 on the 16x16x32 kernel (16-query waves)
    float *part;                      // [B*Hq*Sq][n_ksplit][d + 2]  (o..., m, l), n_ksplit > 1 only
    unsigned *qrot;                   // optional, 16x16x32 kernel: [B*Hq*Sq][d/2] rotated, scaled query pair words
    float scale_log2;                 // log2(e) / sqrt(d)
    int W[kMaxPairs];                 // windows clamped to int32 (kWindowInf = uncut)
    double theta[kMaxPairs];
};

// Arguments of the split-KV decode kernel and its combine step.
struct DecodeArgs {
    const void *q;
    const void *k;
    const void *v;
    float *part;                      // [B*Hq][nsplit][d + 2]  (o..., m, l)
    unsigned *qrot;                   // bf16: [B*Hq][d/2] rotated, scaled query pair words
    void *out;
    unsigned long long *counter;
    int B, Hq, Hkv, group, S, nsplit, n_slabs;
    int cap;                          // key-cache layout: keys per (b, kv head) row of k and v
    // paged key cache: k/v are page pools ([page][Hkv][64-key block]), key block
    // c of sequence b lives in page page_table[b * max_pages + c]; sequence b
    // holds seq_lens[b] keys (device arrays); splits are planned in-kernel
    const int *page_table;
    const int *seq_lens;
    int max_pages, num_pages;
    int split_budget;                 // paged: splits per (kv head, slab) shared by the batch, by length
    int gptj;                         // rotary pairs of q and k: 0 = (p, p + d/2), 1 = (2p, 2p + 1)
    long long pos0;
    float scale_log2;
    int W[kMaxPairs];
    double theta[kMaxPairs];
    int split_start[kMaxSplits + 1];  // key index where each split begins (multiple of 64)
};

// Writes keys into the decode key-cache layout (rotated, 64-key blocks of
// 4-pair planes).
struct KPackArgs {
    const void *k;                    // [B][Hkv][n][d] pre-RoPE keys
    void *kc;                         // the key cache, capacity cap keys per (b, kv head)
    const void *v;                    // nullable: [B][Hkv][n][d] values, copied as rows k_begin.. of vc
    void *vc;                         // the value cache [B][Hkv][cap][d] (with v)
    int B, Hkv, n, cap;
    long long k_begin, pos0;          // key k[.., i, :] is cache key k_begin + i at pos0 + k_begin + i
    int gptj;                         // rotary pairs of k: 0 = (p, p + d/2), 1 = (2p, 2p + 1)
    double theta[kMaxPairs];
};

hipError_t launch_prep_bf16(const PrepArgs &a, int d, hipStream_t s);
hipError_t launch_kpack_bf16(const KPackArgs &a, int d, hipStream_t s);
hipError_t launch_decode_kcache_bf16(const DecodeArgs &a, int d, hipStream_t s);
hipError_t launch_decode_paged_bf16(const DecodeArgs &a, int d, hipStream_t s);

// Writes n tokens of every sequence into a paged key/value cache.
struct PagedWriteArgs {
    const void *k, *v;                // [B][Hkv][n][d] pre-RoPE keys, values
    void *kpool, *vpool;              // [page][Hkv][64-key block] (keys in planes, values in rows)
    const int *page_table;            // [B][max_pages]
    int B, Hkv, n, max_pages, num_pages;
    long long k_begin, pos0;          // token i of the call is token k_begin + i, at pos0 + k_begin + i
    int gptj;                         // rotary pairs of k: 0 = (p, p + d/2), 1 = (2p, 2p + 1)
    double theta[kMaxPairs];
};
hipError_t launch_paged_write_bf16(const PagedWriteArgs &a, int d, hipStream_t s);
hipError_t launch_prep_f32(const PrepArgs &a, int d, hipStream_t s);
hipError_t launch_prefill_bf16(const AttnArgs &a, int d, hipStream_t s);
hipError_t launch_attend_f32(const AttnArgs &a, int d, hipStream_t s);
hipError_t launch_decode_bf16(const DecodeArgs &a, int d, hipStream_t s);
hipError_t launch_fill_zero_u64(unsigned long long *p, hipStream_t s);
// rotates the queries into a.qrot and clears a.counter
hipError_t launch_prefill_qrot(const AttnArgs &a, int d, hipStream_t s);
// Device address of the current GPU's copy of the library's scratch array
// (kNoAllocScratchBytes); looked up once per device and kept.  *ptr = NULL
// when `s` (non-null) belongs to a device other than the current one.
hipError_t noalloc_scratch(hipStream_t s, void **ptr);

}  // namespace atf
